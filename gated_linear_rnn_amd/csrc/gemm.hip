// Gate projections of the RG-LRU (Griffin model-architecture page, section "Real-Gated
// Linear Recurrent Unit (RG-LRU)", Eq. (1)-(2)): z^a = W_a u + b_a and z^x = W_x u + b_x
// for every (batch, time) row, i.e. the dense contraction Z[M, 2D] = U[M, D] [W_a; W_x]^T
// with M = B*T.  This is the one dense contraction of the branch, so it runs on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  The sigmoid gates,
// log-space a_t = exp(c r_t log sigma(Lambda)) (Eq. 3) and sqrt(1 - a_t^2) (Eq. 4) are
// evaluated in the epilogue while the accumulators are still in registers.
//
// Tiling (per workgroup): BM rows of U x BC channels, where the B tile holds the BC rows
// of W_a and the same BC rows of W_x, so each lane ends the K loop holding z^a and z^x of
// the same (row, channel) in matching accumulator slots.  Operands are K-contiguous in
// HBM ([out, in] weights, row-major U), loaded 16 bytes per lane straight into LDS with
// global_load_lds_dwordx4 (no VGPR staging) into a double buffer; rows of 128 bytes are
// XOR-swizzled in 16-byte chunks so the ds_read_b128 operand fetches are conflict-free.
// The workgroup -> tile map groups tiles sharing U and W panels on one XCD for L2 reuse.
#include "rglru_device.h"
#include "kernels.h"

namespace rglru {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

enum : int { kModePlain = 3 };

struct GemmParams {
  const bf16_t* A;
  const bf16_t* A2;
  const bf16_t* B0;
  const bf16_t* B1;
  int M, N, K;
  int lda, ldb, ldc;
  // gate epilogue
  const float* ba;
  const float* bx;
  const float* lam;
  float c;
  float* out0;
  float* out1;
  const bf16_t* u;
  float* h;
  bf16_t* y;
  // plain epilogue
  float* C;
  const float* addend;
};

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Map the linear workgroup id to a (tile_m, tile_n) pair.  Consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs; the remap gives every XCD a contiguous range of
// the grouped tile order, so the tiles one XCD runs together share U and W panels in its L2.
__device__ __forceinline__ void tile_coords(int MT, int NT, int& tm, int& tn) {
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int group = bid / (GM * NT);
  const int first = group * GM;
  const int gsize = min(GM, MT - first);
  const int in = bid - group * GM * NT;
  tm = first + in % gsize;
  tn = in / gsize;
}

template <int BM, int BC, int WM, int WN, int MODE, bool DUAL>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int BNR = 2 * BC;                  // B-tile rows
  constexpr int WTM = BM / WM, WTNR = BNR / WN;
  constexpr int MF = WTM / 32, NF = WTNR / 32;
  constexpr int ROWS = BM + BNR;
  constexpr int STAGE = ROWS * 128;            // bytes per stage (BK = 64 bf16 per row)
  constexpr int QPW = ROWS / 8 / NW;           // DMA instructions per wave per stage
  constexpr int QA = BM / 8 / NW;              // ... of which load U rows
  constexpr int QB1 = (BM + BC) / 8 / NW;      // gate modes: index of the first W_x load
  static_assert(WTM % 32 == 0 && WTNR % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((ROWS / 8) % NW == 0 && (BM / 8) % NW == 0 && ((BM + BC) / 8) % NW == 0, "");
  static_assert(MODE == kModePlain || (BC / WN) % 32 == 0, "");
  static_assert(2 * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int MT = (p.M + BM - 1) / BM;
  const int NT = MODE == kModePlain ? (p.N + BNR - 1) / BNR : (p.N + BC - 1) / BC;
  int tm, tn;
  tile_coords(MT, NT, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * (MODE == kModePlain ? BNR : BC);

  // per-lane source offsets (elements) of this wave's DMA loads
  uint32_t off[QPW];
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
    const int r = (q * NW + wave) * 8 + (lane >> 3);
    const int pchunk = lane & 7;
    if (q < QA) {
      const int gm = min(m0 + r, p.M - 1);
      off[q] = uint32_t(gm) * uint32_t(p.lda) + uint32_t((pchunk ^ ((r >> 1) & 7)) * 8);
    } else {
      const int rb = r - BM;
      int gn;
      if (MODE == kModePlain) gn = min(n0 + rb, p.N - 1);
      else gn = min(n0 + (rb % BC), p.N - 1);
      off[q] = uint32_t(gn) * uint32_t(p.ldb) + uint32_t((pchunk ^ ((rb >> 1) & 7)) * 8);
    }
  }
  const int KT1 = p.K / 64;                    // k tiles per pass
  const int KT = DUAL ? 2 * KT1 : KT1;

  auto issue = [&](int stage, int kt) {
    const bf16_t* abase = (DUAL && kt >= KT1) ? p.A2 : p.A;
    const int kofs = (DUAL && kt >= KT1 ? kt - KT1 : kt) * 64;
    unsigned char* sbase = lds + stage * STAGE;
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
      const bf16_t* base = q < QA ? abase : ((MODE != kModePlain && q >= QB1) ? p.B1 : p.B0);
      const bf16_t* gp = base + off[q] + kofs;
      __builtin_amdgcn_global_load_lds(
          (void*)gp, (void*)(sbase + (q * NW + wave) * 1024), 16, 0, 0);
    }
  };

  // LDS rows of this lane's operand fragments
  int arow[MF], brow[NF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) arow[mf] = wm * WTM + mf * 32 + (lane & 31);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int base;
    if (MODE == kModePlain) {
      base = wn * WTNR + f * 32;
    } else {
      const int half = NF / 2;
      const int g = f / half, jc = f % half;
      base = g * BC + wn * (BC / WN) + jc * 32;
    }
    brow[f] = BM + base + (lane & 31);
  }
  const int swz = ((lane & 31) >> 1) & 7;
  const int khalf = lane >> 5;

  f32x16_t acc[MF][NF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mf][f][v] = 0.f;

  issue(0, 0);
  wait_vmem_all();
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) issue(st ^ 1, kt + 1);
    const unsigned char* sb = lds + st * STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int coff = (((kk * 2 + khalf) ^ swz) * 16);
      bf16x8_t af[MF], bfr[NF];
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
        af[mf] = *reinterpret_cast<const bf16x8_t*>(sb + arow[mf] * 128 + coff);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        bfr[f] = *reinterpret_cast<const bf16x8_t*>(sb + brow[f] * 128 + coff);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[mf][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mf], bfr[f], acc[mf][f], 0, 0, 0);
    }
    wait_vmem_all();
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // accumulator slot v of lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l%32
  const int col = lane & 31;
  const int rbase = 4 * (lane >> 5);
  if (MODE == kModePlain) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = n0 + wn * WTNR + f * 32 + col;
      if (n >= p.N) continue;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * WTM + mf * 32 + 8 * (v >> 2) + rbase + (v & 3);
          if (m < p.M) {
            const size_t o = size_t(m) * p.ldc + n;
            float val = acc[mf][f][v];
            if (p.addend) val += p.addend[o];
            p.C[o] = val;
          }
        }
    }
  } else {
    constexpr int HALF = NF / 2;
#pragma unroll
    for (int jc = 0; jc < HALF; ++jc) {
      const int ch = n0 + wn * (BC / WN) + jc * 32 + col;
      if (ch >= p.N) continue;
      const float ba = p.ba[ch], bx = p.bx[ch];
      const float L = log_sigmoidf(p.lam[ch]);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * WTM + mf * 32 + 8 * (v >> 2) + rbase + (v & 3);
          if (m >= p.M) continue;
          const size_t o = size_t(m) * p.N + ch;
          const Gate g = gate_from_z(acc[mf][jc][v] + ba, acc[mf][jc + HALF][v] + bx, L, p.c);
          if (MODE == kEpiAB) {
            p.out0[o] = g.a;
            p.out1[o] = g.m * g.i;
          } else if (MODE == kEpiRI) {
            p.out0[o] = g.r;
            p.out1[o] = g.i;
          } else {  // kEpiDecode
            const float uu = bf2f(p.u[o]);
            const float hn = fmaf(g.a, p.h[o], (g.m * g.i) * uu);
            p.h[o] = hn;
            p.y[o] = f2bf(hn);
          }
        }
    }
  }
}

// ---------------------------------------------------------------- launchers (bf16)
template <int BM, int BC, int WM, int WN, int MODE, bool DUAL>
static hipError_t run_bf16(const GemmParams& p, hipStream_t s) {
  const int BNR = 2 * BC;
  const int MT = (p.M + BM - 1) / BM;
  const int NT = MODE == kModePlain ? (p.N + BNR - 1) / BNR : (p.N + BC - 1) / BC;
  gemm_bf16_kernel<BM, BC, WM, WN, MODE, DUAL><<<MT * NT, WM * WN * 64, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gate_gemm_bf16(const GateGemmArgs& g, int epi, bool small_m, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.U);
  p.B0 = static_cast<const bf16_t*>(g.Wa);
  p.B1 = static_cast<const bf16_t*>(g.Wx);
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.lda = g.K; p.ldb = g.K; p.ldc = g.N;
  p.ba = g.ba; p.bx = g.bx; p.lam = g.lam; p.c = g.c;
  p.out0 = g.out0; p.out1 = g.out1;
  p.u = static_cast<const bf16_t*>(g.u);
  p.h = g.h;
  p.y = static_cast<bf16_t*>(g.y);
  if (small_m) {
    switch (epi) {
      case kEpiAB: return run_bf16<64, 32, 2, 1, kEpiAB, false>(p, s);
      case kEpiRI: return run_bf16<64, 32, 2, 1, kEpiRI, false>(p, s);
      case kEpiDecode: return run_bf16<64, 32, 2, 1, kEpiDecode, false>(p, s);
    }
  } else {
    switch (epi) {
      case kEpiAB: return run_bf16<256, 128, 2, 2, kEpiAB, false>(p, s);
      case kEpiRI: return run_bf16<256, 128, 2, 2, kEpiRI, false>(p, s);
      case kEpiDecode: return run_bf16<256, 128, 2, 2, kEpiDecode, false>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_plain_gemm_bf16(const PlainGemmArgs& g, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.A);
  p.A2 = static_cast<const bf16_t*>(g.A2);
  p.B0 = static_cast<const bf16_t*>(g.Bm);
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.lda = g.lda; p.ldb = g.ldb; p.ldc = g.ldc;
  p.C = g.C; p.addend = g.addend;
  if (g.A2) return run_bf16<256, 128, 2, 2, kModePlain, true>(p, s);
  return run_bf16<256, 128, 2, 2, kModePlain, false>(p, s);
}

// ---------------------------------------------------------------- fp32 VALU GEMM
// For fp32 I/O (the tiny fp32 workload): C = A B^T (+ addend), 64x64 tiles, 4x4 per
// thread, K-slices of 16 staged transposed in LDS.  Products of fp32 values are exact in
// fp64, so the fp64 accumulation leaves one rounding per output (the weight-gradient
// reductions run over B*T rows).  Latency-bound at these sizes.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ Bm, int M, int N,
                                                       int K, int lda, int ldb, int ldc,
                                                       float* C, const float* addend) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int NT = (N + 63) / 64;
  const int m0 = (blockIdx.x / NT) * 64, n0 = (blockIdx.x % NT) * 64;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const float* ap = A + size_t(min(m0 + lr, M - 1)) * lda + lk;
  const float* bp = Bm + size_t(min(n0 + lr, N - 1)) * ldb + lk;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 av = *reinterpret_cast<const float4*>(ap + k0);
    const float4 bv = *reinterpret_cast<const float4*>(bp + k0);
    __syncthreads();
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(double(a[i]), double(b[j]), acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const size_t o = size_t(m) * ldc + n;
      double v = acc[i][j];
      if (addend) v += addend[o];
      C[o] = float(v);
    }
  }
}

hipError_t launch_plain_gemm_f32(const PlainGemmArgs& g, hipStream_t s) {
  const int blocks = ((g.M + 63) / 64) * ((g.N + 63) / 64);
  gemm_f32_kernel<<<blocks, 256, 0, s>>>(static_cast<const float*>(g.A),
                                         static_cast<const float*>(g.Bm), g.M, g.N, g.K, g.lda,
                                         g.ldb, g.ldc, g.C, g.addend);
  return hipGetLastError();
}

template <int EPI>
__global__ __launch_bounds__(256) void gate_elementwise_f32_kernel(GemmParams p, const float* za,
                                                                   const float* zx) {
  const size_t n = size_t(p.M) * p.N;
  for (size_t o = size_t(blockIdx.x) * blockDim.x + threadIdx.x; o < n;
       o += size_t(gridDim.x) * blockDim.x) {
    const int ch = int(o % p.N);
    const Gate g = gate_from_z(za[o] + p.ba[ch], zx[o] + p.bx[ch], log_sigmoidf(p.lam[ch]), p.c);
    if (EPI == kEpiAB) {
      p.out0[o] = g.a;
      p.out1[o] = g.m * g.i;
    } else if (EPI == kEpiRI) {
      p.out0[o] = g.r;
      p.out1[o] = g.i;
    } else {
      const float* uf = reinterpret_cast<const float*>(p.u);
      float* yf = reinterpret_cast<float*>(p.y);
      const float hn = fmaf(g.a, p.h[o], (g.m * g.i) * uf[o]);
      p.h[o] = hn;
      yf[o] = hn;
    }
  }
}

hipError_t launch_gate_elementwise_f32(const GateGemmArgs& g, const float* za, const float* zx,
                                       int epi, hipStream_t s) {
  GemmParams p{};
  p.M = g.M; p.N = g.N;
  p.ba = g.ba; p.bx = g.bx; p.lam = g.lam; p.c = g.c;
  p.out0 = g.out0; p.out1 = g.out1;
  p.u = static_cast<const bf16_t*>(g.u);
  p.h = g.h;
  p.y = static_cast<bf16_t*>(g.y);
  const size_t n = size_t(g.M) * g.N;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (epi == kEpiAB) gate_elementwise_f32_kernel<kEpiAB><<<int(blocks), 256, 0, s>>>(p, za, zx);
  else if (epi == kEpiRI) gate_elementwise_f32_kernel<kEpiRI><<<int(blocks), 256, 0, s>>>(p, za, zx);
  else gate_elementwise_f32_kernel<kEpiDecode><<<int(blocks), 256, 0, s>>>(p, za, zx);
  return hipGetLastError();
}

}  // namespace rglru
