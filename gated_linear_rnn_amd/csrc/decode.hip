// One decode step of the RG-LRU for bf16 I/O (Griffin model-architecture page, section
// "Real-Gated Linear Recurrent Unit (RG-LRU)", Eq. (1)-(4) at a single time step; the blog
// page "Griffin's Compromise", section "Hawk: Redesigning RNN State with Gates": a step
// reads and writes only the current token and a fixed-size state).
//
// The gate projection of a step is a small-M GEMM (M = batch) whose cost is streaming the
// weights, so its K loop is split S ways to put enough workgroups on the chip: every
// workgroup accumulates z^a and z^x of its (row tile, channel tile) over one K range on the
// matrix cores and writes the raw sums to a partial buffer.  A second kernel adds the S
// partials of each (row, channel) in a fixed order (so the result does not depend on
// scheduling), applies the gates of Eq. (1)-(3) with the biases, and updates the state in
// place: h <- a h + sqrt(1 - a^2) (i u), y = RNE_bf16(h).  The per-channel gate constants
// (biases in the exp2 domain, c log2 sigma(Lambda)) are computed once per channel by the
// first kernel rather than once per (row, channel) by the second.
#include "gemm_core.h"
#include "kernels.h"

namespace rglru {

// 128 rows x 64 channels (64 rows of W_a + the same 64 of W_x), 4 waves of 64 x (32 + 32),
// K steps of 64, double-buffered: 64 KB of LDS, so two workgroups fit on a CU.
typedef GemmCfg<128, 64, 2, 2, false, 64, 2> CfgDecode;

constexpr int kMaxSplits = 8;

int decode_splits(int B, int D) {
  const int MT = (B + CfgDecode::BM - 1) / CfgDecode::BM;
  const int NT = (D + CfgDecode::BC - 1) / CfgDecode::BC;
  const int ksteps = D / CfgDecode::BK;
  // the smallest divisor of the K steps that gives at least one workgroup per CU
  int best = 1;
  for (int s = 1; s <= ksteps && s <= kMaxSplits; ++s) {
    if (ksteps % s) continue;
    best = s;
    if (MT * NT * s >= 256) break;
  }
  return best;
}

size_t decode_partial_bytes(int B, int D) {
  return size_t(decode_splits(B, D)) * 2 * size_t(B) * D * sizeof(float) + 3 * size_t(D) * sizeof(float);
}

// partial[s][0][m][ch] = sum over k in split s of u[m,k] W_a[ch,k]; partial[s][1] for W_x
__global__ __launch_bounds__(CfgDecode::NW * 64, 2) void decode_partial_kernel(DecodeArgs p) {
  typedef CfgDecode C;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int B = p.B, D = p.D, S = p.splits;
  const int MT = (B + C::BM - 1) / C::BM;
  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so that each XCD
  // runs a contiguous range of L = tm + MT (s + S tn): the row tiles that share a W panel
  // then share that XCD's L2, and W streams from the Infinity Cache once per step.
  const int G = gridDim.x;
  const int L = (G & 7) == 0 ? int(blockIdx.x & 7) * (G >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  const int tm = L % MT;
  const int s = (L / MT) % S;
  const int tn = L / (MT * S);
  const int kc = D / S;                            // K columns per split (a multiple of 64)
  const int m0 = tm * C::BM, n0 = tn * C::BC;
  if (tm == 0 && s == 0 && int(threadIdx.x) < C::BC && n0 + int(threadIdx.x) < D) {
    const int ch = n0 + threadIdx.x;
    const GateChan k = gate_chan(p.ba[ch], p.bx[ch], p.lam[ch], p.c);
    p.chan[ch] = k.nba;
    p.chan[D + ch] = k.nbx;
    p.chan[2 * D + ch] = k.cl2;
  }

  TileOperands op;
  op.A = static_cast<const bf16_t*>(p.u) + size_t(s) * kc;
  op.A2 = nullptr;
  op.B0 = static_cast<const bf16_t*>(p.Wa) + size_t(s) * kc;
  op.B1 = static_cast<const bf16_t*>(p.Wx) + size_t(s) * kc;
  op.lda = D; op.ldb = D; op.K = kc;
  op.a_row0 = m0; op.a_rows = B - m0;
  op.b_row0 = n0; op.b_rows = D - n0;
  f32x16_t acc[C::MF][C::NF];
  gemm_mainloop<C, false>(op, lds, lane, wave, acc);

  const size_t BD = size_t(B) * D;
  float* pa = p.partial + size_t(s) * 2 * BD;
  float* px = pa + BD;
  constexpr int HALF = C::NF / 2;
  const int col = lane & 31;
#pragma unroll
  for (int jc = 0; jc < HALF; ++jc) {
    const int ch = n0 + wn * (C::BC / C::WN) + jc * 32 + col;
    if (ch >= D) continue;
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * C::WTM + mf * 32 + acc_row(v, lane);
        if (m >= B) continue;
        // read once, by decode_update_kernel: non-temporal (24.5 -> 24.1 us per step at
        // B = 256, D = 2560)
        __builtin_nontemporal_store(acc[mf][jc][v], pa + size_t(m) * D + ch);
        __builtin_nontemporal_store(acc[mf][jc + HALF][v], px + size_t(m) * D + ch);
      }
  }
}

// Sum the splits in order s = 0..S-1, then the gates and the state update; 4 channels per
// thread (16-byte loads along the channel axis).
__global__ __launch_bounds__(256) void decode_update_kernel(DecodeArgs p) {
  const int B = p.B, D = p.D, S = p.splits;
  const size_t BD = size_t(B) * D;
  const size_t q = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= BD / 4) return;
  const size_t o = q * 4;
  const int ch0 = int(o % D);
  const float* pp = p.partial + o;
  auto ld = [&](int s, int half) { return *reinterpret_cast<const float4*>(pp + (size_t(s) * 2 + half) * BD); };
  auto add = [](float4& acc, const float4& v) { acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w; };
  // up to kMaxSplits partials are loaded before any addition (their loads overlap)
  float4 va[kMaxSplits], vx[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) { va[s] = ld(s, 0); vx[s] = ld(s, 1); }
  float4 za = va[0], zx = vx[0];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S) { add(za, va[s]); add(zx, vx[s]); }
  const float4 h = *reinterpret_cast<const float4*>(p.h + o);
  const float4 u = Io<bf16_t>::load4(static_cast<const bf16_t*>(p.u) + o);
  const float4 nba = *reinterpret_cast<const float4*>(p.chan + ch0);
  const float4 nbx = *reinterpret_cast<const float4*>(p.chan + D + ch0);
  const float4 cl2 = *reinterpret_cast<const float4*>(p.chan + 2 * D + ch0);
  float4 hn;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    GateChan k;
    k.nba = f4get(nba, j);
    k.nbx = f4get(nbx, j);
    k.cl2 = f4get(cl2, j);
    float a, beta;
    gate_fast(f4get(za, j), f4get(zx, j), k, a, beta);
    f4set(hn, j, fmaf(a, f4get(h, j), beta * f4get(u, j)));
  }
  *reinterpret_cast<float4*>(p.h + o) = hn;
  if (p.gate) {   // the recurrent block's GeLU branch multiplies the state before rounding
    const float4 g = Io<bf16_t>::load4(static_cast<const bf16_t*>(p.gate) + o);
    hn.x *= g.x; hn.y *= g.y; hn.z *= g.z; hn.w *= g.w;
  }
  Io<bf16_t>::store4(static_cast<bf16_t*>(p.y) + o, hn);
}

// Small batches (B <= kGemvMaxB = 4): the step's gate projection is a matrix-vector product per
// sequence, bound by streaming W.  One wave per channel reads that channel's W_a and W_x rows
// once (16-byte loads along K), multiplies them with the B rows of u (staged once per
// workgroup in LDS), sums its 64 lanes in a fixed butterfly order, and applies the gates and
// the state update itself: one launch after the conv, no partial sums in memory.  Each lane
// sums its K chunks in order, so repeated calls give identical bits.
constexpr int kGemvMaxB = 4;                  // at B = 6 and 8 the split-K pair is as fast
constexpr int kGemvWaves = 8;                  // channels per workgroup
constexpr int kGemvMaxD = 4096;                // u staging: BB * kGemvMaxD * 2 bytes of LDS

bool decode_uses_gemv(int B, int D) { return B <= kGemvMaxB && D <= kGemvMaxD; }

__device__ __forceinline__ float bfl(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfh(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int BB>
__global__ __launch_bounds__(kGemvWaves * 64) void decode_gemv_kernel(DecodeArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t su[BB * kGemvMaxD];
  const int B = p.B, D = p.D;
  const int lane = threadIdx.x & 63;
  // u [B, D] into LDS, 16 bytes per thread per trip
  const uint4* ug = static_cast<const uint4*>(p.u);
  uint4* ul = reinterpret_cast<uint4*>(su);
  const int n16 = B * D / 8;
  for (int i = threadIdx.x; i < n16; i += blockDim.x) ul[i] = ug[i];
  __syncthreads();
  const int ch = blockIdx.x * kGemvWaves + int(threadIdx.x >> 6);
  if (ch >= D) return;                         // the whole wave: ch is wave-uniform
  const uint4* wa = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(p.Wa) + size_t(ch) * D);
  const uint4* wx = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(p.Wx) + size_t(ch) * D);
  float sa[BB], sx[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) { sa[b] = 0.f; sx[b] = 0.f; }
  for (int c = lane; c < D / 8; c += 64) {     // 8 consecutive k per 16-byte chunk
    const uint4 va = wa[c], vx = wx[c];
    const float a8[8] = {bfl(va.x), bfh(va.x), bfl(va.y), bfh(va.y), bfl(va.z), bfh(va.z), bfl(va.w), bfh(va.w)};
    const float x8[8] = {bfl(vx.x), bfh(vx.x), bfl(vx.y), bfh(vx.y), bfl(vx.z), bfh(vx.z), bfl(vx.w), bfh(vx.w)};
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      if (b < B) {
        const uint4 vu = ul[size_t(b) * (D / 8) + c];
        const float u8[8] = {bfl(vu.x), bfh(vu.x), bfl(vu.y), bfh(vu.y), bfl(vu.z), bfh(vu.z), bfl(vu.w), bfh(vu.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sa[b] = fmaf(a8[e], u8[e], sa[b]);
          sx[b] = fmaf(x8[e], u8[e], sx[b]);
        }
      }
    }
  }
  // butterfly over the 64 lanes; a + b == b + a, so every lane ends with the same sums
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      sa[b] += __shfl_xor(sa[b], off);
      sx[b] += __shfl_xor(sx[b], off);
    }
  if (lane >= B) return;
  float za = 0.f, zx = 0.f;
#pragma unroll
  for (int b = 0; b < BB; ++b)
    if (b == lane) { za = sa[b]; zx = sx[b]; }
  const int b = lane;
  const GateChan k = gate_chan(p.ba[ch], p.bx[ch], p.lam[ch], p.c);
  float a, beta;
  gate_fast(za, zx, k, a, beta);
  const size_t o = size_t(b) * D + ch;
  const float hn = fmaf(a, p.h[o], beta * bf2f(su[o]));
  p.h[o] = hn;
  const float yv = p.gate ? hn * bf2f(static_cast<const bf16_t*>(p.gate)[o]) : hn;
  static_cast<bf16_t*>(p.y)[o] = f2bf(yv);
}

hipError_t launch_decode_bf16(const DecodeArgs& a_in, hipStream_t s) {
  DecodeArgs a = a_in;
  if (decode_uses_gemv(a.B, a.D)) {
    const int blocks = (a.D + kGemvWaves - 1) / kGemvWaves;
    switch (a.B) {
      case 1: decode_gemv_kernel<1><<<blocks, kGemvWaves * 64, 0, s>>>(a); break;
      case 2: decode_gemv_kernel<2><<<blocks, kGemvWaves * 64, 0, s>>>(a); break;
      default: decode_gemv_kernel<4><<<blocks, kGemvWaves * 64, 0, s>>>(a); break;
    }
    return hipGetLastError();
  }
  a.splits = decode_splits(a.B, a.D);
  a.chan = a.partial + size_t(a.splits) * 2 * size_t(a.B) * a.D;
  const int MT = (a.B + CfgDecode::BM - 1) / CfgDecode::BM;
  const int NT = (a.D + CfgDecode::BC - 1) / CfgDecode::BC;
  decode_partial_kernel<<<MT * NT * a.splits, CfgDecode::NW * 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t quads = size_t(a.B) * a.D / 4;
  decode_update_kernel<<<int((quads + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rglru
