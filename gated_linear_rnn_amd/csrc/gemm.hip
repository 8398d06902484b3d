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
#include "gemm_core.h"
#include "kernels.h"

namespace rglru {

// kModePlain: fp32 C (+ addend).  kModeInProj: the two input linears of the recurrent
// block, N = 2R columns; columns [0, R) are written to C16 as bf16 (the branch input p),
// columns [R, 2R) go through GeLU and to G16 as bf16.  kModeOut: bf16 C16.
// kModeGeglu (gate tile: B0 rows and the same B1 rows paired): the first layer of the
// gated MLP block, C16 = RNE(GeLU(A B0^T) * (A B1^T)).  kModeQkv: the projections of the
// local-MQA block, N = D + 256 columns: q = columns [0, D) to C16 (ldc D), k = the next 128
// to G16, v = the last 128 to V16 (ldc 128); q and k are rotated (RoPE) before rounding.
enum : int { kModePlain = 3, kModeInProj = 4, kModeOut = 5, kModeGeglu = 6, kModeQkv = 7 };

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
  const bf16_t* u;   // fp32 decode (as raw bytes of the io type)
  float* h;
  bf16_t* y;
  // plain epilogue
  float* C;
  const float* addend;
  float* C2;          // kModePlain: rows m >= m_split go to C2 (row m - m_split)
  int m_split;
  bf16_t* C16;        // kModeInProj (p), kModeOut, kModeQkv (q)
  bf16_t* G16;        // kModeInProj (GeLU branch), kModeQkv (k)
  bf16_t* V16;        // kModeQkv (v)
  int split;          // kModeInProj: R; kModeQkv: D
  int T, pos0;        // kModeQkv: row m is at position pos0 + m % T
  // kModeOut / kModePlain tail split: workgroups [0, tail_first) compute whole tiles (the tiles
  // [0, tail_first) of the grouped order); the remaining tiles are each computed by
  // tail_split workgroups over equal K ranges into fp32 partials at tail_ws, which
  // tail_fixup_kernel adds and rounds.  Without a split tail_first = MT * NT.
  int tail_first, tail_split;
  float* tail_ws;
};

// Tile (tm, tn) of position L in the grouped order: groups of GM = 8 row tiles, and within a
// group all column tiles, so consecutive tiles share row and column panels.
__device__ __forceinline__ void grouped_tile(int L, int MT, int NT, int& tm, int& tn) {
  constexpr int GM = 8;
  const int group = L / (GM * NT);
  const int first = group * GM;
  const int gsize = min(GM, MT - first);
  const int in = L - group * GM * NT;
  tm = first + in % gsize;
  tn = in / gsize;
}

// Number of CUs the tail split plans for (MI355X); another count only makes it less exact.
constexpr int kPlanCUs = 256;

// RoPE angle of position pos and frequency theta (radians per position), in turns reduced
// to [-1/2, 1/2]: the product and the reduction in fp64, so that large positions keep full
// fp32 accuracy; the hardware sine and cosine (v_sin_f32 / v_cos_f32) take turns.
__device__ __forceinline__ float rope_turns(int pos, double theta_turns) {
  const double a = double(pos) * theta_turns;
  return float(a - rint(a));
}

// Map the workgroup id to a tile (tm, tn) and, for tail-split workgroups, a K part.
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs; the remap gives
// every XCD a contiguous range of the grouped tile order, so the tiles one XCD runs together
// share panels in its L2 (in the split tail, the parts of a tile stay on one XCD too).
__device__ __forceinline__ void tile_coords(int MT, int NT, int first, int split, int& tm, int& tn,
                                            int& part, int& L) {
  part = 0;
  if (int(blockIdx.x) < first) {
    L = blockIdx.x;
    if ((first & 7) == 0) L = (L & 7) * (first >> 3) + (L >> 3);
  } else {
    const int nt = int(gridDim.x) - first;
    int q = int(blockIdx.x) - first;
    if ((nt & 7) == 0) q = (q & 7) * (nt >> 3) + (q >> 3);
    L = first + q / split;
    part = q % split;
  }
  grouped_tile(L, MT, NT, tm, tn);
}

template <class C, int MODE, bool DUAL>
__global__ __launch_bounds__(C::NW * 64, C::NW >= 8 ? 2 : 1) void gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int MT = (p.M + C::BM - 1) / C::BM;
  constexpr bool kPlainTile = C::PLAIN;   // plain tiles span BNR columns, gate tiles BC channels
  const int NT = kPlainTile ? (p.N + C::BNR - 1) / C::BNR : (p.N + C::BC - 1) / C::BC;
  int tm, tn, part, L;
  tile_coords(MT, NT, p.tail_first, p.tail_split, tm, tn, part, L);
  const bool tail = (MODE == kModeOut || MODE == kModePlain || MODE == kEpiAB || MODE == kEpiRI) &&
                    int(blockIdx.x) >= p.tail_first;
  const int m0 = tm * C::BM;
  const int n0 = tn * (kPlainTile ? C::BNR : C::BC);
  const int kc = tail ? p.K / p.tail_split : p.K;

  TileOperands op;
  op.A = p.A + size_t(part) * kc; op.A2 = p.A2 ? p.A2 + size_t(part) * kc : nullptr;
  op.B0 = p.B0 + size_t(part) * kc; op.B1 = p.B1 ? p.B1 + size_t(part) * kc : nullptr;
  op.lda = p.lda; op.ldb = p.ldb; op.K = kc;
  op.a_row0 = m0; op.a_rows = p.M - m0;
  op.b_row0 = n0; op.b_rows = p.N - n0;
  f32x16_t acc[C::MF][C::NF];
  gemm_mainloop<C, DUAL>(op, lds, lane, wave, acc);

  // ---------------------------------------------------------------- epilogue
  const int col = lane & 31;
  if (tail) {
    // fp32 partial of this K part: the whole tile, row-major [BM][BNR], columns in B-tile
    // row order (gate tiles: the BC z^a channels, then the BC z^x channels)
    float* dst = p.tail_ws + (size_t(L - p.tail_first) * p.tail_split + part) * (C::BM * C::BNR);
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      constexpr int HF = C::NF / 2;
      const int bcol = C::PLAIN ? wn * C::WTNR + f * 32 + col
                                : (f / HF) * C::BC + wn * (C::BC / C::WN) + (f % HF) * 32 + col;
#pragma unroll
      for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * C::WTM + mf * 32 + acc_row(v, lane);
          dst[r * C::BNR + bcol] = acc[mf][f][v];
        }
    }
  } else if (MODE == kModePlain) {
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      const int n = n0 + wn * C::WTNR + f * 32 + col;
      if (n >= p.N) continue;
#pragma unroll
      for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * C::WTM + mf * 32 + acc_row(v, lane);
          if (m < p.M) {
            const size_t o = size_t(m) * p.ldc + n;
            float val = acc[mf][f][v];
            if (p.addend) val += p.addend[o];
            if (m < p.m_split) p.C[o] = val;
            else p.C2[size_t(m - p.m_split) * p.ldc + n] = val;
          }
        }
    }
  } else if (MODE == kModeInProj || MODE == kModeOut || MODE == kModeQkv) {
    // bf16 output through LDS: each wave rounds its 128 x 64 block into its own 16 KB of
    // the (now idle) operand ring, then writes whole 128-byte row segments, 16 bytes per
    // lane.  In LDS a block row is 8 chunks of 16 bytes; rows r and r + 4 (the two lane
    // halves of one accumulator write) sit 64 bytes apart in the bank space (chunk XOR 4)
    // so the 2-byte writes of the two halves use disjoint banks.
    static_assert(C::WTNR == 64 && C::NW * C::WTM * C::WTNR * 2 <= C::LDS_BYTES, "staging");
    __syncthreads();   // every wave is done reading the last operand stage
    bf16_t* st = reinterpret_cast<bf16_t*>(lds) + wave * (C::WTM * C::WTNR);
    const int nb = n0 + wn * C::WTNR;   // first column of the wave's block
    // the split is a multiple of 64 and so is nb: a block lies on one side of it
    const bool gelu_side = MODE == kModeInProj && nb >= p.split;
    // kModeQkv: q and k columns are rotated; column pairs (2i, 2i+1) sit in lanes l, l^1
    const bool rot = MODE == kModeQkv && nb < p.split + 128;
    double theta[C::NF];   // 10000^(-2i/128) / (2 pi) turns per position, i = pair index
    float c1[C::NF], s1[C::NF];   // the rotation by one position
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      theta[f] = exp2(-double(((nb + f * 32 + col) & 127) >> 1) * (13.287712379549449 / 64.0)) *
                 0.15915494309189533577;
      const float t1 = float(theta[f]);
      c1[f] = __builtin_amdgcn_cosf(t1);
      s1[f] = __builtin_amdgcn_sinf(t1);
    }
    // Accumulator slots 4g .. 4g+3 are four consecutive rows (positions): the angle of the
    // first is evaluated exactly (fp64 reduction), the next three by rotating it one
    // position at a time, unless the group straddles the end of a sequence.
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
      for (int f = 0; f < C::NF; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rbase = mf * 32 + 8 * g + 4 * (lane >> 5);
          const int pm = (m0 + wm * C::WTM + rbase) % (MODE == kModeQkv ? p.T : 1);
          float cs = 1.f, sn = 0.f;
          if (rot) {
            const float turns = rope_turns(p.pos0 + pm, theta[f]);
            sn = __builtin_amdgcn_sinf(turns);
            cs = __builtin_amdgcn_cosf(turns);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int v = 4 * g + j, r = rbase + j;
            const int chunk = (f * 4 + (col >> 3)) ^ (((r >> 2) & 1) << 2);
            float val = acc[mf][f][v];
            if (MODE == kModeQkv) {
              const float other = __int_as_float(
                  __builtin_amdgcn_mov_dpp(__float_as_int(val), 0xB1, 0xF, 0xF, false));   // lane ^ 1
              if (rot) {
                if (j > 0) {
                  if (pm + j < p.T) {
                    const float cn = fmaf(cs, c1[f], -sn * s1[f]);
                    sn = fmaf(sn, c1[f], cs * s1[f]);
                    cs = cn;
                  } else {     // the group runs into the next sequence(s)
                    const float turns = rope_turns(p.pos0 + (pm + j) % p.T, theta[f]);
                    sn = __builtin_amdgcn_sinf(turns);
                    cs = __builtin_amdgcn_cosf(turns);
                  }
                }
                val = (col & 1) ? fmaf(other, sn, val * cs) : fmaf(val, cs, -other * sn);
              }
            }
            st[r * 64 + chunk * 8 + (col & 7)] = f2bf(gelu_side ? gelu_fast(val) : val);
          }
        }
    // LDS operations of a wave complete in order; the fence keeps the compiler from
    // moving the reads below above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // destination of the block: base pointer (indexed by the global column) and row stride
    bf16_t* dst0 = gelu_side ? p.G16 - p.split : p.C16;
    int ldc = p.ldc;
    if (MODE == kModeQkv && nb >= p.split) {
      dst0 = nb < p.split + 128 ? p.G16 - p.split : p.V16 - (p.split + 128);
      ldc = 128;
    }
#pragma unroll
    for (int it = 0; it < C::WTM / 8; ++it) {
      const int r = it * 8 + (lane >> 3), ck = lane & 7;
      const int m = m0 + wm * C::WTM + r, n = nb + ck * 8;
      const uint4 val = *reinterpret_cast<const uint4*>(st + r * 64 + ((ck ^ (((r >> 2) & 1) << 2)) * 8));
      if (m < p.M && n < p.N) *reinterpret_cast<uint4*>(dst0 + size_t(m) * ldc + n) = val;
    }
  } else if (MODE == kModeGeglu) {
    // The workgroup's 256 x 128 bf16 output tile is assembled in LDS (the idle operand
    // ring), then written as whole 256-byte rows, 16 bytes per lane.  A tile row is 16
    // chunks of 16 bytes; rows r and r + 4 (the two lane halves of one accumulator write)
    // sit 64 bytes apart in the bank space (chunk XOR 4) so their 2-byte writes use
    // disjoint banks.
    constexpr int HALF = C::NF / 2;
    constexpr int CPR16 = C::BC / 8;                   // 16-byte chunks per tile row
    static_assert(C::BM * C::BC * 2 <= C::LDS_BYTES && CPR16 == 16, "staging");
    __syncthreads();   // every wave is done reading the last operand stage
    bf16_t* st = reinterpret_cast<bf16_t*>(lds);
#pragma unroll
    for (int jc = 0; jc < HALF; ++jc) {
      const int cl = wn * (C::BC / C::WN) + jc * 32 + col;   // channel within the tile
#pragma unroll
      for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * C::WTM + mf * 32 + acc_row(v, lane);
          const int chunk = (cl >> 3) ^ (((r >> 2) & 1) << 2);
          const float val = gelu_fast(acc[mf][jc][v]) * acc[mf][jc + HALF][v];
          st[r * C::BC + chunk * 8 + (cl & 7)] = f2bf(val);
        }
    }
    __syncthreads();
    constexpr int kIters = C::BM * CPR16 / (C::NW * 64);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int idx = it * C::NW * 64 + int(threadIdx.x);
      const int r = idx / CPR16, ck = idx % CPR16;
      const int m = m0 + r, n = n0 + ck * 8;
      const uint4 val = *reinterpret_cast<const uint4*>(st + r * C::BC + ((ck ^ (((r >> 2) & 1) << 2)) * 8));
      // non-temporal: a whole-row hand-off to the output linear (15 us of 1.63 ms at the
      // training shape)
      if (m < p.M && n < p.N) {
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4v{val.x, val.y, val.z, val.w},
                                    reinterpret_cast<u32x4v*>(p.C16 + size_t(m) * p.ldc + n));
      }
    }
  } else {
    constexpr int HALF = C::NF / 2;
#pragma unroll
    for (int jc = 0; jc < HALF; ++jc) {
      const int ch = n0 + wn * (C::BC / C::WN) + jc * 32 + col;
      if (ch >= p.N) continue;
      const GateChan k = gate_chan(p.ba[ch], p.bx[ch], p.lam[ch], p.c);
#pragma unroll
      for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * C::WTM + mf * 32 + acc_row(v, lane);
          if (m >= p.M) continue;
          const size_t o = size_t(m) * p.N + ch;
          const float za = acc[mf][jc][v], zx = acc[mf][jc + HALF][v];
          // (r, i) or (a, beta) are read once by the scan that follows: stored with the
          // non-temporal hint, so they do not leave dirty lines in the Infinity Cache whose
          // write-back would compete with that scan's reads (112 -> 98 us for the scan
          // right after the gate GEMM at 8 x 2048 x 2560)
          if (MODE == kEpiRI) {
            float r, i;
            gate_fast_ri(za, zx, k, r, i);
            __builtin_nontemporal_store(r, p.out0 + o);
            __builtin_nontemporal_store(i, p.out1 + o);
          } else {  // kEpiAB
            float a, beta;
            gate_fast(za, zx, k, a, beta);
            __builtin_nontemporal_store(a, p.out0 + o);
            __builtin_nontemporal_store(beta, p.out1 + o);
          }
        }
    }
  }
}

// ---------------------------------------------------------------- launchers (bf16)
// 256 x 256 tiles, 8 waves of 128 x 64, BK = 64, double-buffered.
typedef GemmCfg<256, 128, 2, 4, false, 64, 2> CfgGate;
typedef GemmCfg<256, 128, 2, 4, true, 64, 2> CfgPlain;

// Tail split: the tiles of the last, partly filled round (R of them) are each computed by
// S workgroups over K / S, so that they take about ceil(S R / CUs) / S of a full tile's
// time instead of one.  S in {2, 3, 4} with (K / BK) % S == 0 minimising that (the
// smaller S on a tie, fewer partials); 1 when nothing is gained (no partial round, or a
// last round so full that no split fits it in fewer tile times).
static void plan_tail(int tiles, int ksteps, int& first, int& split) {
  const int R = tiles % kPlanCUs;
  first = tiles;
  split = 1;
  if (R == 0) return;
  double best = 1.0;
  for (int sp = 2; sp <= 4; ++sp) {
    if (ksteps % sp) continue;
    const double cost = double((sp * R + kPlanCUs - 1) / kPlanCUs) / sp;
    if (cost < best - 1e-9) {
      best = cost;
      split = sp;
      first = tiles - R;
    }
  }
}

size_t out_gemm_tail_bytes(int M, int N, int K) {
  typedef GemmCfg<256, 128, 2, 4, true, 64, 2> C;
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BNR - 1) / C::BNR);
  int first, split;
  plan_tail(tiles, K / C::BK, first, split);
  return split > 1 ? size_t(tiles - first) * split * C::BM * C::BNR * sizeof(float) : 0;
}
size_t plain_gemm_tail_bytes(int M, int N, int K) { return out_gemm_tail_bytes(M, N, K); }
size_t gate_gemm_tail_bytes(int M, int N, int K) {
  typedef GemmCfg<256, 128, 2, 4, false, 64, 2> C;
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BC - 1) / C::BC);
  int first, split;
  plan_tail(tiles, K / C::BK, first, split);
  return split > 1 ? size_t(tiles - first) * split * C::BM * C::BNR * sizeof(float) : 0;
}

// The split tail's fixup: sum the S partials of each element in order, round to bf16,
// store inside the matrix.  One thread per 8 consecutive columns of a tile row.
template <class C>
__global__ __launch_bounds__(256) void tail_fixup_kernel(GemmParams p, int MT, int NT) {
  constexpr int CH = C::BNR / 8;
  const size_t per_tile = size_t(C::BM) * CH;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int ntail = MT * NT - p.tail_first;
  if (idx >= per_tile * ntail) return;
  const int i = int(idx / per_tile);
  const int r = int(idx % per_tile) / CH, ck = int(idx % per_tile) % CH;
  int tm, tn;
  grouped_tile(p.tail_first + i, MT, NT, tm, tn);
  const int m = tm * C::BM + r, n = tn * C::BNR + ck * 8;
  if (m >= p.M || n >= p.N) return;
  const float* src = p.tail_ws + size_t(i) * p.tail_split * (C::BM * C::BNR) + r * C::BNR + ck * 8;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = src[e];
  for (int sp = 1; sp < p.tail_split; ++sp)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += src[size_t(sp) * (C::BM * C::BNR) + e];
  uint4 w;
  w.x = uint32_t(f2bf(v[0])) | (uint32_t(f2bf(v[1])) << 16);
  w.y = uint32_t(f2bf(v[2])) | (uint32_t(f2bf(v[3])) << 16);
  w.z = uint32_t(f2bf(v[4])) | (uint32_t(f2bf(v[5])) << 16);
  w.w = uint32_t(f2bf(v[6])) | (uint32_t(f2bf(v[7])) << 16);
  *reinterpret_cast<uint4*>(p.C16 + size_t(m) * p.ldc + n) = w;
}

// The same fixup for the fp32 plain mode: partials summed in order, the addend added last
// (as the untiled epilogue does), rows past m_split written to C2.
template <class C>
__global__ __launch_bounds__(256) void tail_fixup_f32_kernel(GemmParams p, int MT, int NT) {
  constexpr int CH = C::BNR / 8;
  const size_t per_tile = size_t(C::BM) * CH;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int ntail = MT * NT - p.tail_first;
  if (idx >= per_tile * ntail) return;
  const int i = int(idx / per_tile);
  const int r = int(idx % per_tile) / CH, ck = int(idx % per_tile) % CH;
  int tm, tn;
  grouped_tile(p.tail_first + i, MT, NT, tm, tn);
  const int m = tm * C::BM + r, n0 = tn * C::BNR + ck * 8;
  if (m >= p.M || n0 >= p.N) return;
  const float* src = p.tail_ws + size_t(i) * p.tail_split * (C::BM * C::BNR) + r * C::BNR + ck * 8;
  float4 v0 = *reinterpret_cast<const float4*>(src), v1 = *reinterpret_cast<const float4*>(src + 4);
  for (int sp = 1; sp < p.tail_split; ++sp) {
    const float4 a0 = *reinterpret_cast<const float4*>(src + size_t(sp) * (C::BM * C::BNR));
    const float4 a1 = *reinterpret_cast<const float4*>(src + size_t(sp) * (C::BM * C::BNR) + 4);
    v0.x += a0.x; v0.y += a0.y; v0.z += a0.z; v0.w += a0.w;
    v1.x += a1.x; v1.y += a1.y; v1.z += a1.z; v1.w += a1.w;
  }
  const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float* dst = m < p.m_split ? p.C + size_t(m) * p.ldc : p.C2 + size_t(m - p.m_split) * p.ldc;
  const float* add = p.addend ? p.addend + size_t(m) * p.ldc : nullptr;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int n = n0 + e;
    if (n < p.N) dst[n] = add ? v[e] + add[n] : v[e];
  }
}

// The same fixup for the gate modes: z^a and z^x of each (row, channel) summed over the
// parts in order, then the gate epilogue of the whole tiles.
template <class C, int MODE>
__global__ __launch_bounds__(256) void tail_fixup_gate_kernel(GemmParams p, int MT, int NT) {
  const size_t per_tile = size_t(C::BM) * C::BC;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int ntail = MT * NT - p.tail_first;
  if (idx >= per_tile * ntail) return;
  const int i = int(idx / per_tile);
  const int r = int(idx % per_tile) / C::BC, c = int(idx % per_tile) % C::BC;
  int tm, tn;
  grouped_tile(p.tail_first + i, MT, NT, tm, tn);
  const int m = tm * C::BM + r, ch = tn * C::BC + c;
  if (m >= p.M || ch >= p.N) return;
  const float* src = p.tail_ws + size_t(i) * p.tail_split * (C::BM * C::BNR) + r * C::BNR + c;
  float za = src[0], zx = src[C::BC];
  for (int sp = 1; sp < p.tail_split; ++sp) {
    za += src[size_t(sp) * (C::BM * C::BNR)];
    zx += src[size_t(sp) * (C::BM * C::BNR) + C::BC];
  }
  const GateChan k = gate_chan(p.ba[ch], p.bx[ch], p.lam[ch], p.c);
  const size_t o = size_t(m) * p.N + ch;
  if (MODE == kEpiRI) {
    float rr, ii;
    gate_fast_ri(za, zx, k, rr, ii);
    __builtin_nontemporal_store(rr, p.out0 + o);
    __builtin_nontemporal_store(ii, p.out1 + o);
  } else {
    float a, beta;
    gate_fast(za, zx, k, a, beta);
    __builtin_nontemporal_store(a, p.out0 + o);
    __builtin_nontemporal_store(beta, p.out1 + o);
  }
}

template <class C, int MODE, bool DUAL>
static hipError_t run_bf16(GemmParams p, hipStream_t s) {
  const int MT = (p.M + C::BM - 1) / C::BM;
  const int NT = C::PLAIN ? (p.N + C::BNR - 1) / C::BNR : (p.N + C::BC - 1) / C::BC;
  static_assert(C::PLAIN == (MODE == kModePlain || MODE == kModeInProj || MODE == kModeOut ||
                             MODE == kModeQkv),
                "plain-tile modes run on plain configurations");
  const int tiles = MT * NT;
  p.tail_first = tiles;
  p.tail_split = 1;
  if ((MODE == kModeOut || MODE == kModePlain || MODE == kEpiAB || MODE == kEpiRI) && p.tail_ws)
    plan_tail(tiles, p.K / C::BK, p.tail_first, p.tail_split);
  const int grid = p.tail_first + (tiles - p.tail_first) * p.tail_split;
  gemm_bf16_kernel<C, MODE, DUAL><<<grid, C::NW * 64, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.tail_split == 1) return e;
  if (MODE == kEpiAB || MODE == kEpiRI) {
    const size_t gthreads = size_t(tiles - p.tail_first) * C::BM * C::BC;
    tail_fixup_gate_kernel<C, MODE><<<int((gthreads + 255) / 256), 256, 0, s>>>(p, MT, NT);
    return hipGetLastError();
  }
  const size_t threads = size_t(tiles - p.tail_first) * C::BM * (C::BNR / 8);
  if (MODE == kModePlain) tail_fixup_f32_kernel<C><<<int((threads + 255) / 256), 256, 0, s>>>(p, MT, NT);
  else tail_fixup_kernel<C><<<int((threads + 255) / 256), 256, 0, s>>>(p, MT, NT);
  return hipGetLastError();
}

hipError_t launch_gate_gemm_bf16(const GateGemmArgs& g, int epi, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.U);
  p.B0 = static_cast<const bf16_t*>(g.Wa);
  p.B1 = static_cast<const bf16_t*>(g.Wx);
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.lda = g.K; p.ldb = g.K; p.ldc = g.N;
  p.ba = g.ba; p.bx = g.bx; p.lam = g.lam; p.c = g.c;
  p.out0 = g.out0; p.out1 = g.out1;
  p.tail_ws = g.tail_ws;
  switch (epi) {
    case kEpiAB: return run_bf16<CfgGate, kEpiAB, false>(p, s);
    case kEpiRI: return run_bf16<CfgGate, kEpiRI, false>(p, s);
  }
  return hipErrorInvalidValue;   // the bf16 decode step has its own kernels (decode.hip)
}

hipError_t launch_plain_gemm_bf16(const PlainGemmArgs& g, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.A);
  p.A2 = static_cast<const bf16_t*>(g.A2);
  p.B0 = static_cast<const bf16_t*>(g.Bm);
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.lda = g.lda; p.ldb = g.ldb; p.ldc = g.ldc;
  p.C = g.C; p.addend = g.addend;
  p.C2 = g.C2;
  p.m_split = g.m_split > 0 ? g.m_split : g.M;
  p.tail_ws = g.tail_ws;
  if (g.A2) return run_bf16<CfgPlain, kModePlain, true>(p, s);
  return run_bf16<CfgPlain, kModePlain, false>(p, s);
}

hipError_t launch_block_gemm_bf16(const BlockGemmArgs& g, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.A);
  p.B0 = static_cast<const bf16_t*>(g.Bm);
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.lda = g.K; p.ldb = g.K; p.ldc = g.ldc;
  p.C16 = static_cast<bf16_t*>(g.C);
  p.G16 = static_cast<bf16_t*>(g.G);
  p.split = g.split;
  if (g.G) return run_bf16<CfgPlain, kModeInProj, false>(p, s);
  p.tail_ws = g.tail_ws;
  return run_bf16<CfgPlain, kModeOut, false>(p, s);
}

hipError_t launch_qkv_gemm_bf16(const QkvGemmArgs& g, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.A);
  p.B0 = static_cast<const bf16_t*>(g.W);
  p.M = g.M; p.N = g.D + 256; p.K = g.D;
  p.lda = g.D; p.ldb = g.D; p.ldc = g.D;
  p.C16 = static_cast<bf16_t*>(g.q);
  p.G16 = static_cast<bf16_t*>(g.k);
  p.V16 = static_cast<bf16_t*>(g.v);
  p.split = g.D; p.T = g.T; p.pos0 = g.pos0;
  return run_bf16<CfgPlain, kModeQkv, false>(p, s);
}

hipError_t launch_geglu_gemm_bf16(const GegluGemmArgs& g, hipStream_t s) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.A);
  p.B0 = static_cast<const bf16_t*>(g.W1);
  p.B1 = static_cast<const bf16_t*>(g.W2);
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.lda = g.K; p.ldb = g.K; p.ldc = g.N;
  p.C16 = static_cast<bf16_t*>(g.H);
  return run_bf16<CfgGate, kModeGeglu, false>(p, s);
}

// ---------------------------------------------------------------- fp32 VALU GEMM
// For fp32 I/O (the tiny fp32 workload): C = A B^T (+ addend), TM x TM tiles, 4x4 per thread,
// K-slices of 16 staged transposed in LDS.  Products of fp32 values are exact in fp64, so the
// fp64 accumulation leaves one rounding per output (the weight-gradient reductions run over
// B*T rows); each output is summed over k in order by one thread, so the tile size does not
// change any bit.  Latency-bound at these sizes: 64 x 64 tiles (256 threads) when they give
// the GPU at least one workgroup per CU, else 32 x 32 tiles (64 threads, four times the
// workgroups).  With B1 (grid.y = 2) the same launch also computes C1 = A B1^T: the two gate
// projections of the fp32 forward in one launch.
template <int TM, int R>
__global__ __launch_bounds__((TM / R) * (TM / R)) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    int M, int N, int K, int lda, int ldb, int ldc, float* C0, float* C1,
    const float* addend) {
  // TM x TM output tile, R x R outputs per thread
  constexpr int TX = TM / R, NTH = TX * TX, LPT = TM * 4 / NTH;
  static_assert(LPT >= 1 && TM * 4 % NTH == 0, "loader");
  __shared__ float As[16][TM + 4];
  __shared__ float Bs[16][TM + 4];
  const float* Bm = blockIdx.y ? B1 : B0;
  float* C = blockIdx.y ? C1 : C0;
  const int tid = threadIdx.x;
  const int tx = tid % TX, ty = tid / TX;
  const int NT = (N + TM - 1) / TM;
  const int m0 = (blockIdx.x / NT) * TM, n0 = (blockIdx.x % NT) * TM;
  const float* ap[LPT];
  const float* bp[LPT];
  int lr[LPT], lk[LPT];
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int idx = tid + q * NTH;
    lr[q] = idx >> 2;
    lk[q] = (idx & 3) * 4;
    ap[q] = A + size_t(min(m0 + lr[q], M - 1)) * lda + lk[q];
    bp[q] = Bm + size_t(min(n0 + lr[q], N - 1)) * ldb + lk[q];
  }
  double acc[R][R] = {};
  // The next k-step's operands are loaded into registers while the current one is
  // computed, so each step waits on loads issued a whole step earlier.
  float4 av[LPT], bv[LPT];
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    av[q] = *reinterpret_cast<const float4*>(ap[q]);
    bv[q] = *reinterpret_cast<const float4*>(bp[q]);
  }
  for (int k0 = 0; k0 < K; k0 += 16) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
      As[lk[q] + 0][lr[q]] = av[q].x; As[lk[q] + 1][lr[q]] = av[q].y;
      As[lk[q] + 2][lr[q]] = av[q].z; As[lk[q] + 3][lr[q]] = av[q].w;
      Bs[lk[q] + 0][lr[q]] = bv[q].x; Bs[lk[q] + 1][lr[q]] = bv[q].y;
      Bs[lk[q] + 2][lr[q]] = bv[q].z; Bs[lk[q] + 3][lr[q]] = bv[q].w;
    }
    __syncthreads();
    if (k0 + 16 < K) {
#pragma unroll
      for (int q = 0; q < LPT; ++q) {
        av[q] = *reinterpret_cast<const float4*>(ap[q] + k0 + 16);
        bv[q] = *reinterpret_cast<const float4*>(bp[q] + k0 + 16);
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[R], b[R];
#pragma unroll
      for (int i = 0; i < R; ++i) a[i] = As[k][ty * R + i];
#pragma unroll
      for (int j = 0; j < R; ++j) b[j] = Bs[k][tx * R + j];
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[i][j] = fma(double(a[i]), double(b[j]), acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int m = m0 + ty * R + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int n = n0 + tx * R + j;
      if (n >= N) continue;
      const size_t o = size_t(m) * ldc + n;
      double v = acc[i][j];
      if (addend) v += addend[o];
      C[o] = float(v);
    }
  }
}

static hipError_t launch_gemm_f32(const float* A, const float* B0, const float* B1, int M, int N,
                                  int K, int lda, int ldb, int ldc, float* C0, float* C1,
                                  const float* addend, hipStream_t s) {
  const int pairs = B1 ? 2 : 1;
  // the largest tile that still gives every CU a workgroup (each output sums k in order
  // whatever the tile, so the choice does not change the result)
  auto tiles = [&](int tm) { return long((M + tm - 1) / tm) * ((N + tm - 1) / tm) * pairs; };
  if (tiles(64) >= 256) {
    const dim3 grid(((M + 63) / 64) * ((N + 63) / 64), pairs);
    gemm_f32_kernel<64, 4><<<grid, 256, 0, s>>>(A, B0, B1, M, N, K, lda, ldb, ldc, C0, C1, addend);
  } else if (tiles(32) >= 256) {
    const dim3 grid(((M + 31) / 32) * ((N + 31) / 32), pairs);
    gemm_f32_kernel<32, 4><<<grid, 64, 0, s>>>(A, B0, B1, M, N, K, lda, ldb, ldc, C0, C1, addend);
  } else {
    const dim3 grid(((M + 15) / 16) * ((N + 15) / 16), pairs);
    gemm_f32_kernel<16, 2><<<grid, 64, 0, s>>>(A, B0, B1, M, N, K, lda, ldb, ldc, C0, C1, addend);
  }
  return hipGetLastError();
}

hipError_t launch_plain_gemm_f32(const PlainGemmArgs& g, hipStream_t s) {
  return launch_gemm_f32(static_cast<const float*>(g.A), static_cast<const float*>(g.Bm), nullptr,
                         g.M, g.N, g.K, g.lda, g.ldb, g.ldc, g.C, nullptr, g.addend, s);
}

hipError_t launch_gemm_f32_pair(const float* A, const float* B0, const float* B1, int M, int N,
                                int K, float* C0, float* C1, hipStream_t s) {
  return launch_gemm_f32(A, B0, B1, M, N, K, K, K, N, C0, C1, nullptr, s);
}

template <int EPI>
__global__ __launch_bounds__(256) void gate_elementwise_f32_kernel(GemmParams p, const float* za,
                                                                   const float* zx) {
  const size_t n = size_t(p.M) * p.N;
  for (size_t o = size_t(blockIdx.x) * blockDim.x + threadIdx.x; o < n;
       o += size_t(gridDim.x) * blockDim.x) {
    const int ch = int(o % p.N);
    const float r = sigmoidf_stable(za[o] + p.ba[ch]);
    const float i = sigmoidf_stable(zx[o] + p.bx[ch]);
    if (EPI == kEpiRI) {
      p.out0[o] = r;
      p.out1[o] = i;
      continue;
    }
    // a and m in fp64, then one rounding: an fp32 exponential's small rounding bias in a
    // would compound through the recurrence
    const GateAmD g = gate_am(r, double(log_sigmoidf(p.lam[ch])), p.c);
    if (EPI == kEpiAB) {
      p.out0[o] = float(g.a);
      p.out1[o] = float(g.m * double(i));
    } else {
      const float* uf = reinterpret_cast<const float*>(p.u);
      float* yf = reinterpret_cast<float*>(p.y);
      const float hn = float(fma(g.a, double(p.h[o]), (g.m * double(i)) * double(uf[o])));
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
