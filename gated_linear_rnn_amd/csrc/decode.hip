// One decode step of the RG-LRU for bf16 I/O (Griffin model-architecture page, section
// "Real-Gated Linear Recurrent Unit (RG-LRU)", Eq. (1)-(4) at a single time step; the blog
// page "Griffin's Compromise", section "Hawk: Redesigning RNN State with Gates": a step
// reads and writes only the current token and a fixed-size state).
//
// After the conv launch (which shifts the conv history in place and writes u), one kernel
// does the rest of the step.  Its gate projection is a small-M GEMM (M = batch): z^a = u W_a^T
// and z^x = u W_x^T over K = D.  A workgroup owns BM rows x BC channels over ALL of K, so the
// gates and the state update run in its own epilogue and nothing but the state and y leaves
// the kernel.  Its 8 waves split the K loop; no operand element is used by two waves, so the
// fragments go from memory through a private LDS ring of each wave into registers (16
// bytes per lane, v_mfma_f32_16x16x32_bf16, fp32 accumulation).  The 8 partial tiles
// are then summed in LDS in one fixed tree order, so a step's result does not depend on
// scheduling and repeated steps give identical bits.
//
// The tile shape is picked per (B, D) from BM in {16, 32, 64} and BC in {16, 32, 40, 64}
// with MF + NF <= 9 (the LDS ring takes 16 (MF + NF) KB):
// each workgroup reads (BM + 2 BC) rows of K, and the pick minimises that per round of 256
// CUs (B = 256, D = 2560: 64 x 40 tiles, 256 workgroups).
#include "kernels.h"
#include "rglru_device.h"

namespace rglru {

typedef __bf16 bf16x8d_t __attribute__((ext_vector_type(8)));
typedef float f32x4d_t __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 8;
constexpr int kDecSlice = 32;   // K per MFMA (16x16x32)

// MF 16-row blocks of u rows, NF 16-row blocks of the B tile (BC = 8 NF channels: rows
// 0..BC-1 of the B tile are W_a rows, BC..2BC-1 the same W_x rows).
template <int MF, int NF>
struct DecCfg {
  static constexpr int BM = 16 * MF, NB = 16 * NF, BC = NB / 2;
  static constexpr int TILE = MF * NF * 4 * 64;          // floats of one wave's partial tile
  static constexpr int ZLD = NB + 1;                      // row stride of the summed tile
  static constexpr int SLOT = (MF + NF) * 1024;           // bytes of one slice's fragments
  static constexpr int RING = kDecWaves * 2 * SLOT / 4;   // floats: two slots per wave
  static constexpr int RED0 = 4 * TILE > BM * ZLD ? 4 * TILE : BM * ZLD;
  static constexpr int RED = RING > RED0 ? RING : RED0;
  static constexpr int LDS = (RED + 3 * BC) * 4;
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Wait until at most N of this wave's vector-memory operations are pending (the builtin
// informs the compiler's own wait-count tracking; the asm keeps LDS reads behind it).
template <int N>
__device__ __forceinline__ void dec_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void dec_wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int MF, int NF>
__global__ __launch_bounds__(kDecWaves * 64, 1) void decode_fused_kernel(DecodeArgs p) {
  typedef DecCfg<MF, NF> C;
  __shared__ __attribute__((aligned(16))) float dsm[C::LDS / 4];
  float* red = dsm;                                      // 4 partial tiles (fragment order)
  float* zt = dsm;                                       // then [BM][ZLD]: the summed z
  float* chan = dsm + C::RED;                            // [3][BC] gate constants
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int B = p.B, D = p.D;
  const int ntn = D / C::BC;
  // consecutive workgroups take consecutive channel tiles of one row tile: the round-robin
  // dispatch then spreads the channel tiles (the W stream) over the XCDs, and every XCD
  // reads u of the row tile once into its L2
  const int tn = int(blockIdx.x) % ntn, tm = int(blockIdx.x) / ntn;
  const int m0 = tm * C::BM, ch0 = tn * C::BC;

  // Everything the epilogue reads from memory is loaded before the K loop, so its latency
  // hides behind the loop: the per-channel gate parameters, and h and u of this thread's
  // EPT elements (element e = threadIdx.x + 512 i of the tile, row e / BC, channel e % BC).
  constexpr int EPT = (C::BM * C::BC + kDecWaves * 64 - 1) / (kDecWaves * 64);
  float ba = 0.f, bx = 0.f, lam = 0.f;
  if (int(threadIdx.x) < C::BC) {
    const int ch = ch0 + threadIdx.x;
    ba = p.ba[ch];
    bx = p.bx[ch];
    lam = p.lam[ch];
  }
  const bf16_t* u = static_cast<const bf16_t*>(p.u);
  const bf16_t* gate = static_cast<const bf16_t*>(p.gate);
  float hv[EPT], uv[EPT], gv[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x + i * kDecWaves * 64;
    const int m = m0 + e / C::BC;
    const bool ok = e < C::BM * C::BC && m < B;
    const size_t o = size_t(ok ? m : 0) * D + ch0 + (ok ? e % C::BC : 0);
    hv[i] = ok ? p.h[o] : 0.f;
    uv[i] = ok ? bf2f(u[o]) : 0.f;
    gv[i] = ok && gate ? bf2f(gate[o]) : 1.f;
  }

  // this lane's operand rows and k offset within a slice
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const bf16_t* arow[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int m = min(m0 + 16 * mf + r16, B - 1);        // rows past B: computed, not stored
    arow[mf] = static_cast<const bf16_t*>(p.u) + size_t(m) * D + kq;
  }
  const bf16_t* brow[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const int q = 16 * nf + r16;
    const bf16_t* W = static_cast<const bf16_t*>(q < C::BC ? p.Wa : p.Wx);
    brow[nf] = W + size_t(ch0 + (q < C::BC ? q : q - C::BC)) * D + kq;
  }

  f32x4d_t acc[MF][NF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = f32x4d_t{0.f, 0.f, 0.f, 0.f};

  // this wave's K slices: [s0, s1) of D / 32.  Each slice's fragments come through a
  // private two-slot LDS ring of this wave: global_load_lds puts lane l's 16 bytes at
  // lane l's place in the slot, so the lane reads back exactly its own fragment data; no
  // other wave touches the slot, so only this wave's own wait counts are needed.  While the
  // matrix cores multiply slice j, slices j+1 and j+2 are in flight.
  const int KS = D / kDecSlice;
  const int s0 = wave * KS / kDecWaves, s1 = (wave + 1) * KS / kDecWaves;
  const int n = s1 - s0;
  unsigned char* ring = reinterpret_cast<unsigned char*>(dsm) + wave * 2 * C::SLOT;
  struct Frags {
    bf16x8d_t a[MF], b[NF];
  };
  auto dma = [&](int j, int slot) {
    const int k = (s0 + j) * kDecSlice;
    unsigned char* dst = ring + slot * C::SLOT;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
      __builtin_amdgcn_global_load_lds((void*)(arow[mf] + k), (void*)(dst + mf * 1024), 16, 0, 0);
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
      __builtin_amdgcn_global_load_lds((void*)(brow[nf] + k), (void*)(dst + (MF + nf) * 1024), 16, 0, 0);
  };
  auto frags = [&](int slot, Frags& f) {
    const unsigned char* src = ring + slot * C::SLOT + lane * 16;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) f.a[mf] = *reinterpret_cast<const bf16x8d_t*>(src + mf * 1024);
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) f.b[nf] = *reinterpret_cast<const bf16x8d_t*>(src + (MF + nf) * 1024);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mf], f.b[nf], acc[mf][nf], 0, 0, 0);
  };
  if (n > 0) dma(0, 0);
  if (n > 1) dma(1, 1);
  for (int j = 0; j < n; ++j) {
    // slice j has landed once only the slice issued after it (j + 1, if any) is pending
    if (j + 1 < n) dec_wait_vm<MF + NF>();
    else dec_wait_vm<0>();
    Frags f;
    frags(j & 1, f);
    dec_wait_lds();                                   // the slot is free again
    if (j + 2 < n) dma(j + 2, j & 1);
    mma(f);
  }
  __syncthreads();                                    // every ring is drained: LDS is reused

  // fixed-order tree: ((w0 + w4) + (w2 + w6)) + ((w1 + w5) + (w3 + w7))
  auto frag_off = [&](int mf, int nf, int i) { return ((mf * NF + nf) * 4 + i) * 64 + lane; };
#pragma unroll
  for (int half = 4; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      float* dst = red + (wave - half) * C::TILE;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[frag_off(mf, nf, i)] = acc[mf][nf][i];
    }
    __syncthreads();
    if (wave < half) {
      const float* src = red + wave * C::TILE;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mf][nf][i] += src[frag_off(mf, nf, i)];
    }
    __syncthreads();
  }
  // the sum, row-major: output (row 4 (lane / 16) + i, column lane % 16) of each 16x16 block
  if (wave == 0) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          zt[(16 * mf + 4 * (lane >> 4) + i) * C::ZLD + 16 * nf + r16] = acc[mf][nf][i];
  }
  __syncthreads();

  // epilogue: gates, h <- a h + sqrt(1 - a^2) i u, y = RNE(h) (or RNE(h g) with a gate)
  if (int(threadIdx.x) < C::BC) {
    const GateChan k = gate_chan(ba, bx, lam, p.c);
    chan[threadIdx.x] = k.nba;
    chan[C::BC + threadIdx.x] = k.nbx;
    chan[2 * C::BC + threadIdx.x] = k.cl2;
  }
  __syncthreads();
  bf16_t* y = static_cast<bf16_t*>(p.y);
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x + i * kDecWaves * 64;
    const int r = e / C::BC, c = e % C::BC;
    const int m = m0 + r;
    if (e >= C::BM * C::BC || m >= B) continue;
    const size_t o = size_t(m) * D + ch0 + c;
    GateChan k;
    k.nba = chan[c];
    k.nbx = chan[C::BC + c];
    k.cl2 = chan[2 * C::BC + c];
    float a, beta;
    gate_fast(zt[r * C::ZLD + c], zt[r * C::ZLD + C::BC + c], k, a, beta);
    const float hn = fmaf(a, hv[i], beta * uv[i]);
    p.h[o] = hn;
    y[o] = f2bf(gate ? hn * gv[i] : hn);
  }
}

namespace {

struct DecPick {
  int mf, nf;
};

// (BM + 2 BC) rows of K per workgroup, times the rounds of 256 CUs the grid needs
DecPick decode_pick(int B, int D) {
  const int mfs[3] = {4, 2, 1};
  const int nfs[4] = {5, 8, 4, 2};
  DecPick best{1, 2};
  long best_cost = -1, best_wg = 0;
  for (int mf : mfs) {
    const int bm = 16 * mf;
    if (mf > 1 && bm / 2 >= B) continue;                 // a smaller BM already covers B
    for (int nf : nfs) {
      const int bc = 8 * nf;
      if (D % bc || mf + nf > 9) continue;             // the LDS ring: 16 (MF + NF) KB
      const long wg = long((B + bm - 1) / bm) * (D / bc);
      const long cost = ((wg + 255) / 256) * (bm + 2 * bc);
      if (best_cost < 0 || cost < best_cost || (cost == best_cost && wg < best_wg)) {
        best = {mf, nf};
        best_cost = cost;
        best_wg = wg;
      }
    }
  }
  return best;
}

template <int MF, int NF>
hipError_t launch_pick(const DecodeArgs& a, hipStream_t s) {
  typedef DecCfg<MF, NF> C;
  const int grid = ((a.B + C::BM - 1) / C::BM) * (a.D / C::BC);
  decode_fused_kernel<MF, NF><<<grid, kDecWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int MF>
hipError_t launch_mf(const DecodeArgs& a, int nf, hipStream_t s) {
  switch (nf) {
    case 2: return launch_pick<MF, 2>(a, s);
    case 4: return launch_pick<MF, 4>(a, s);
    case 5: return launch_pick<MF, 5>(a, s);
    default:
      if constexpr (MF == 1) return launch_pick<MF, 8>(a, s);
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const DecPick k = decode_pick(a.B, a.D);
  switch (k.mf) {
    case 1: return launch_mf<1>(a, k.nf, s);
    case 2: return launch_mf<2>(a, k.nf, s);
    default: return launch_mf<4>(a, k.nf, s);
  }
}

}  // namespace rglru
