// One generation step of the local multi-query attention block with a bounded key/value
// cache (Griffin model-architecture page, section "Local sliding-window attention": the
// cache is limited to the window).  The cache of a sequence has W slots; slot j holds the
// rotated key and the value of the most recent position p with p % W == j, so at position
// pos the live slots are 0 .. min(pos, W - 1): contiguous, and all inside the window.
//
// Kernels of a bf16 step:
//   splitk_partial_kernel    the projections of the B new tokens are small-M GEMMs whose
//                            cost is streaming the weights: the K loop is split S ways on
//                            the matrix cores into fp32 partial sums (used twice: q/k/v and
//                            the output projection)
//   qkv_finish_kernel        adds the S partials in a fixed order, applies RoPE to q and k
//                            at the sequence's position and writes q, and k, v into the
//                            cache slot pos % W
//   decode_attn_kernel       one workgroup per (sequence, group of 32 heads): the 8 waves
//                            split the live slots in 64-slot tiles; each wave computes
//                            S^T = K Q^T (K read straight from the cache into registers as
//                            the A operand, one head per lane), the online softmax, and
//                            O^T = V^T P^T (V^T transposed through the wave's own LDS
//                            region); the 8 partial (max, sum, O) triples are merged in LDS
//   out_finish_kernel        adds the output projection's partials, rounds to bf16
// fp32 I/O uses the fp64-accumulating VALU GEMM (one "partial"), the same finish kernels
// and a one-thread-per-head fp64 attention kernel.
#include "gemm_core.h"
#include "kernels.h"

namespace rglru {

constexpr int kDhD = 128;

// ---------------------------------------------------------------- split-K projections
// 128 rows x 128 columns per workgroup, 4 waves of 64 x 64, K steps of 64, double-buffered.
typedef GemmCfg<128, 64, 2, 2, true, 64, 2> CfgSplitK;
constexpr int kMaxSplitK = 8;

int splitk_splits(int M, int N, int K) {
  const int MT = (M + CfgSplitK::BM - 1) / CfgSplitK::BM;
  const int NT = (N + CfgSplitK::BNR - 1) / CfgSplitK::BNR;
  const int ksteps = K / CfgSplitK::BK;
  int best = 1;
  for (int s = 1; s <= ksteps && s <= kMaxSplitK; ++s) {
    if (ksteps % s) continue;
    best = s;
    if (MT * NT * s >= 256) break;
  }
  return best;
}

// partial[s][m][n] = sum over the K range of split s of A[m,k] Bm[n,k]
__global__ __launch_bounds__(CfgSplitK::NW * 64, 2) void splitk_partial_kernel(
    const bf16_t* A, const bf16_t* Bm, int M, int N, int K, int S, float* partial) {
  typedef CfgSplitK C;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int MT = (M + C::BM - 1) / C::BM;
  // consecutive ids go round-robin over the 8 XCDs: renumber so one XCD runs a contiguous
  // range of L = tm + MT (s + S tn), i.e. the row tiles and splits of one column block
  const int G = gridDim.x;
  const int L = (G & 7) == 0 ? int(blockIdx.x & 7) * (G >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  const int tm = L % MT, s = (L / MT) % S, tn = L / (MT * S);
  const int kc = K / S;
  const int m0 = tm * C::BM, n0 = tn * C::BNR;
  TileOperands op;
  op.A = A + size_t(s) * kc;
  op.A2 = nullptr;
  op.B0 = Bm + size_t(s) * kc;
  op.B1 = nullptr;
  op.lda = K; op.ldb = K; op.K = kc;
  op.a_row0 = m0; op.a_rows = M - m0;
  op.b_row0 = n0; op.b_rows = N - n0;
  f32x16_t acc[C::MF][C::NF];
  gemm_mainloop<C, false>(op, lds, lane, wave, acc);
  float* ps = partial + size_t(s) * M * N;
  const int col = lane & 31;
#pragma unroll
  for (int f = 0; f < C::NF; ++f) {
    const int n = n0 + wn * C::WTNR + f * 32 + col;
    if (n >= N) continue;
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * C::WTM + mf * 32 + acc_row(v, lane);
        if (m < M) ps[size_t(m) * N + n] = acc[mf][f][v];
      }
  }
}

hipError_t launch_splitk_bf16(const void* A, const void* Bm, int M, int N, int K, int S, float* partial,
                             hipStream_t st) {
  const int MT = (M + CfgSplitK::BM - 1) / CfgSplitK::BM;
  const int NT = (N + CfgSplitK::BNR - 1) / CfgSplitK::BNR;
  splitk_partial_kernel<<<MT * NT * S, CfgSplitK::NW * 64, 0, st>>>(
      static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(Bm), M, N, K, S, partial);
  return hipGetLastError();
}

size_t splitk_partial_bytes(int M, int N, int K) {
  return size_t(splitk_splits(M, N, K)) * M * N * sizeof(float);
}

// position of sequence b (negative positions are taken as 0)
__device__ __forceinline__ int seq_pos(const int* pos, int b) { return max(pos[b], 0); }

// ---------------------------------------------------------------- q/k/v finish
// One thread per (sequence, column pair): the S partials of columns 2c, 2c+1 added in order;
// q (c < D/2) and k pairs rotated at the sequence's position; q to qbuf [B, D], k and v to
// slot pos % W of the caches [B, W, 128].
template <typename IO>
__global__ __launch_bounds__(256) void qkv_finish_kernel(const float* partial, int S, int B, int D,
                                                         const int* pos, int W, IO* qbuf,
                                                         IO* kcache, IO* vcache) {
  const int N = D + 2 * kDhD, NP = N / 2;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= size_t(B) * NP) return;
  const int b = int(idx / NP), c = int(idx % NP);
  double e = 0.0, o = 0.0;   // the fp32 partials summed in fp64, in split order
  for (int s = 0; s < S; ++s) {
    const float* ps = partial + (size_t(s) * B + b) * N + 2 * c;
    e += ps[0];
    o += ps[1];
  }
  const int p = seq_pos(pos, b);
  const int col = 2 * c;
  if (col < D + kDhD) {      // q or k: RoPE pair (2i, 2i+1), i = (col % 128) / 2
    const int i = (col & (kDhD - 1)) >> 1;
    const double theta = exp2(-double(i) * (13.287712379549449 / 64.0));   // 10000^(-2i/128)
    double sn, cs;
    sincos(double(p) * theta, &sn, &cs);
    const double re = e * cs - o * sn, ro = e * sn + o * cs;
    e = re;
    o = ro;
  }
  IO* dst;
  if (col < D) {
    dst = qbuf + size_t(b) * D + col;
  } else {
    const size_t slot = (size_t(b) * W + (p % W)) * kDhD;
    dst = col < D + kDhD ? kcache + slot + (col - D) : vcache + slot + (col - D - kDhD);
  }
  Io<IO>::store1(dst, float(e));
  Io<IO>::store1(dst + 1, float(o));
}

// out [B, N] = RNE_io(sum of the S partials), in a fixed order
template <typename IO>
__global__ __launch_bounds__(256) void out_finish_kernel(const float* partial, int S, int B, int N,
                                                         IO* out) {
  const size_t n = size_t(B) * N;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  float acc = partial[idx];
  for (int s = 1; s < S; ++s) acc += partial[size_t(s) * n + idx];
  Io<IO>::store1(out + idx, acc);
}

hipError_t launch_splitk_out_bf16(const float* partial, int S, int M, int N, void* out, hipStream_t st) {
  const size_t n = size_t(M) * N;
  out_finish_kernel<bf16_t><<<int((n + 255) / 256), 256, 0, st>>>(partial, S, M, N, static_cast<bf16_t*>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------- attention (bf16)
constexpr int kSlotTile = 64;
constexpr int kWaveVt = kDhD * kSlotTile * 2;   // one wave's V^T tile: 16 KB

// V^T row d, position pos (the B-operand key permutation: bits 2 and 3 swapped), 16-byte
// chunks XOR-swizzled by row
__device__ __forceinline__ int dvt_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }
__device__ __forceinline__ int dvt_off(int d, int pos) {
  return d * 128 + (((pos >> 3) ^ ((d >> 1) ^ (d >> 4))) & 7) * 16 + (pos & 7) * 2;
}

__global__ __launch_bounds__(512) void decode_attn_bf16_kernel(const bf16_t* qbuf, const bf16_t* kcache,
                                                               const bf16_t* vcache, const int* pos,
                                                               int B, int H, int W, float scale_log2,
                                                               bf16_t* attn) {
  // LDS: 8 wave-private V^T tiles (128 KB); after the walk, the same bytes hold the 8
  // waves' partial O (32 heads x 128 dims fp32 each), then m and l
  __shared__ __attribute__((aligned(1024))) unsigned char lds[8 * kWaveVt + 8 * 64 * 2 * 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HG = (H + 31) / 32;
  const int b = blockIdx.x / HG, hg = blockIdx.x % HG;
  const int D = H * kDhD;
  const int half = lane >> 5, col = lane & 31;
  const int head = hg * 32 + col;
  const bool hok = head < H;
  const int p = seq_pos(pos, b);
  const int nlive = min(p + 1, W);
  const int ntiles = (nlive + kSlotTile - 1) / kSlotTile;
  const bf16_t* kb_ = kcache + size_t(b) * W * kDhD;
  const bf16_t* vb_ = vcache + size_t(b) * W * kDhD;

  bf16x8_t qf[8];
  {
    const bf16_t* qrow = qbuf + size_t(b) * D + size_t(min(head, H - 1)) * kDhD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * ks);
      if (!hok) qf[ks] = bf16x8_t{};
    }
  }
  f32x16_t acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.f;
  float m_run = -1e30f, l_run = 0.f;
  unsigned char* vt = lds + wave * kWaveVt;

  for (int kt = wave; kt < ntiles; kt += 8) {
    const int j0 = kt * kSlotTile;
    // V tile -> wave-private V^T (keys 2 kp, 2 kp + 1 per lane pair of positions)
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int kp = it * 4 + (lane >> 4), dc = lane & 15;
      const int j = j0 + 2 * kp;
      const uint4 a = *reinterpret_cast<const uint4*>(vb_ + size_t(min(j, nlive - 1)) * kDhD + dc * 8);
      const uint4 c = *reinterpret_cast<const uint4*>(vb_ + size_t(min(j + 1, nlive - 1)) * kDhD + dc * 8);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
      const int ps = dvt_pos(2 * kp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (aw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (cw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(vt + dvt_off(dc * 8 + e, ps)) = lo | (hi << 16);
      }
    }
    // the V loads stay ahead of the K loads: with both in flight at once the wave needs more
    // than its 256 registers and spills
    __builtin_amdgcn_sched_barrier(0);
    // S^T = K Q^T, K rows straight from the cache
    f32x16_t acc_s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_s[kb][v] = 0.f;
      const bf16_t* krow = kb_ + size_t(min(j0 + kb * 32 + col, nlive - 1)) * kDhD + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ks);
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc_s[kb], 0, 0, 0);
      }
    }
    float mx = -1e30f;
    const int jl = nlive - j0 - 4 * half;            // slots j with j - 4 half < jl are live
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kb * 32 + 8 * (v >> 2) + (v & 3);
        const float sc = j < jl ? acc_s[kb][v] * scale_log2 : -INFINITY;
        acc_s[kb][v] = sc;
        mx = fmaxf(mx, sc);
      }
    {
      const WaveHalves mh = wave_halves(mx);       // this lane's and the partner lane's max
      mx = fmaxf(mh.lo, mh.hi);
    }
    const bool bump = mx > m_run + 8.f;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
    }
    float lsum = 0.f;
    bf16x8_t pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(acc_s[kb][v] - m_run);
        lsum += e;
        pf[kb * 2 + (v >> 3)][v & 7] = (__bf16)e;
      }
    l_run += lsum;
    // the wave's V^T writes are complete before its reads (in-order LDS queue); the
    // fences keep the compiler from reordering them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vt + dvt_off(d, 16 * j + 8 * half));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], acc_o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the 8 waves: O_w [32 heads][128 dims] fp32 over the V^T regions, then m, l
  __syncthreads();
  float* osh = reinterpret_cast<float*>(lds);                 // [8][32][128]
  float* msh = reinterpret_cast<float*>(lds + 8 * kWaveVt);   // [8][64]: m per lane
  float* lsh = msh + 8 * 64;                                  // [8][64]: l per lane
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        osh[(wave * 32 + col) * kDhD + db * 32 + 8 * g + 4 * half + r] = acc_o[db][4 * g + r];
  msh[wave * 64 + lane] = m_run;
  lsh[wave * 64 + lane] = l_run;
  __syncthreads();
  // 32 heads x 128 dims, 8 per thread
  const int hq = tid >> 4, d0 = (tid & 15) * 8;
  float mw[8], m = -1e30f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    mw[w] = msh[w * 64 + hq];
    m = fmaxf(m, mw[w]);
  }
  float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float sc = __builtin_amdgcn_exp2f(mw[w] - m);
    l = fmaf(lsh[w * 64 + hq] + lsh[w * 64 + hq + 32], sc, l);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(osh[(w * 32 + hq) * kDhD + d0 + e], sc, o[e]);
  }
  const int hd = hg * 32 + hq;
  if (hd < H) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint4 w4;
    w4.x = uint32_t(f2bf(o[0] * inv)) | (uint32_t(f2bf(o[1] * inv)) << 16);
    w4.y = uint32_t(f2bf(o[2] * inv)) | (uint32_t(f2bf(o[3] * inv)) << 16);
    w4.z = uint32_t(f2bf(o[4] * inv)) | (uint32_t(f2bf(o[5] * inv)) << 16);
    w4.w = uint32_t(f2bf(o[6] * inv)) | (uint32_t(f2bf(o[7] * inv)) << 16);
    *reinterpret_cast<uint4*>(attn + size_t(b) * D + size_t(hd) * kDhD + d0) = w4;
  }
}

// fp32 I/O: one thread per (sequence, head), fp64 softmax over the live slots
__global__ __launch_bounds__(128) void decode_attn_f32_kernel(const float* qbuf, const float* kcache,
                                                              const float* vcache, const int* pos,
                                                              int B, int H, int W, float* attn) {
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= size_t(B) * H) return;
  const int b = int(idx / H), h = int(idx % H);
  const int D = H * kDhD;
  const int nlive = min(seq_pos(pos, b) + 1, W);
  const float* q = qbuf + size_t(b) * D + size_t(h) * kDhD;
  const float* kb = kcache + size_t(b) * W * kDhD;
  const float* vb = vcache + size_t(b) * W * kDhD;
  const double scale = 1.0 / sqrt(double(kDhD));
  double mx = -1e300;
  for (int j = 0; j < nlive; ++j) {
    double dot = 0.0;
    for (int d = 0; d < kDhD; ++d) dot = fma(double(q[d]), double(kb[size_t(j) * kDhD + d]), dot);
    mx = fmax(mx, dot * scale);
  }
  double acc[kDhD];
  for (int d = 0; d < kDhD; ++d) acc[d] = 0.0;
  double l = 0.0;
  for (int j = 0; j < nlive; ++j) {
    double dot = 0.0;
    for (int d = 0; d < kDhD; ++d) dot = fma(double(q[d]), double(kb[size_t(j) * kDhD + d]), dot);
    const double w = exp(dot * scale - mx);
    l += w;
    for (int d = 0; d < kDhD; ++d) acc[d] = fma(w, double(vb[size_t(j) * kDhD + d]), acc[d]);
  }
  float* o = attn + size_t(b) * D + size_t(h) * kDhD;
  for (int d = 0; d < kDhD; ++d) o[d] = float(acc[d] / l);
}

// ---------------------------------------------------------------- the step
size_t mqa_decode_partial_bytes(int B, int D) {
  const int N1 = D + 2 * kDhD;
  const size_t a = splitk_partial_bytes(B, N1, D);
  const size_t c = splitk_partial_bytes(B, D, D);
  return a > c ? a : c;
}

hipError_t launch_mqa_decode(const MqaDecodeArgs& a, hipStream_t st) {
  const int B = a.B, D = a.D, H = D / kDhD, N1 = D + 2 * kDhD;
  const int NP = N1 / 2;
  const size_t pairs = size_t(B) * NP;
  hipError_t e;
  if (a.bf16) {
    const int S1 = splitk_splits(B, N1, D);
    e = launch_splitk_bf16(a.x, a.Wqkv, B, N1, D, S1, a.partial, st);
    if (e != hipSuccess) return e;
    qkv_finish_kernel<bf16_t><<<int((pairs + 255) / 256), 256, 0, st>>>(
        a.partial, S1, B, D, a.pos, a.window, static_cast<bf16_t*>(a.qbuf),
        static_cast<bf16_t*>(a.kcache), static_cast<bf16_t*>(a.vcache));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int HG = (H + 31) / 32;
    decode_attn_bf16_kernel<<<B * HG, 512, 0, st>>>(
        static_cast<const bf16_t*>(a.qbuf), static_cast<const bf16_t*>(a.kcache),
        static_cast<const bf16_t*>(a.vcache), a.pos, B, H, a.window,
        float(1.4426950408889634 / sqrt(double(kDhD))), static_cast<bf16_t*>(a.attn));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int S2 = splitk_splits(B, D, D);
    e = launch_splitk_bf16(a.attn, a.Wo, B, D, D, S2, a.partial, st);
    if (e != hipSuccess) return e;
    return launch_splitk_out_bf16(a.partial, S2, B, D, a.out, st);
  }
  PlainGemmArgs pa{};
  pa.A = a.x; pa.Bm = a.Wqkv; pa.M = B; pa.N = N1; pa.K = D; pa.lda = D; pa.ldb = D; pa.ldc = N1;
  pa.C = a.partial;
  if ((e = launch_plain_gemm_f32(pa, st)) != hipSuccess) return e;
  qkv_finish_kernel<float><<<int((pairs + 255) / 256), 256, 0, st>>>(
      a.partial, 1, B, D, a.pos, a.window, static_cast<float*>(a.qbuf), static_cast<float*>(a.kcache),
      static_cast<float*>(a.vcache));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t nh = size_t(B) * H;
  decode_attn_f32_kernel<<<int((nh + 127) / 128), 128, 0, st>>>(
      static_cast<const float*>(a.qbuf), static_cast<const float*>(a.kcache),
      static_cast<const float*>(a.vcache), a.pos, B, H, a.window, static_cast<float*>(a.attn));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  PlainGemmArgs po{};
  po.A = a.attn; po.Bm = a.Wo; po.M = B; po.N = D; po.K = D; po.lda = D; po.ldb = D; po.ldc = D;
  po.C = static_cast<float*>(a.out);
  return launch_plain_gemm_f32(po, st);
}

}  // namespace rglru
