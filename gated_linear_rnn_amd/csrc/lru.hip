// The RG-LRU layer in one kernel for bf16 I/O: the gate projections of Eq. (1)-(2) on the
// matrix cores, the log-space gates of Eq. (3), and the diagonal recurrence of Eq. (4)
// evaluated in the GEMM epilogue (Griffin model-architecture page, section "Real-Gated
// Linear Recurrent Unit (RG-LRU)").  The input is u, the conv output.
//
// A workgroup owns 256 consecutive time steps of one sequence x 128 channels.  After the
// K loop each lane holds z^a and z^x for one channel and 64 of the tile's time steps (16
// groups of 4 consecutive steps; the partner lane l^32 holds the interleaved groups, the
// other row half lives in the other wave row).  The epilogue turns them into a_t and
// beta_t u_t, scans each group to an affine summary (A = prod a, H), combines the summaries
// along time - partner lanes by a lane exchange, the two wave rows through LDS - and
// chains tiles along time with the decoupled look-back of the chunked scan (the blog page
// "Griffin's Compromise", "Term explanation: Parallel scan").  Only y (bf16) and h_T leave
// the kernel: a_t and beta_t never touch HBM.
//
// With a gate tensor g (the recurrent block's GeLU branch, same layout as u) the kernel
// writes RNE(h_t g_t) instead of RNE(h_t): the g tile is fetched into LDS right behind the
// u tile (the gated kernel takes 146 KB of LDS instead of 128 KB; one workgroup per CU
// either way) and lands during the first pass; the second pass multiplies each state by
// its g before rounding.
//
// Tiles of one chain (sequence b, channel tile) must be started in time order: every
// workgroup takes a ticket from the counter of its group g = blockIdx % G; group g owns a
// contiguous range of the chains in a blocked order (blocks of bw sequences, channel tile
// by channel tile), so all tiles of a chain share one counter, and tickets enumerate its
// tiles time-level by time-level.  A tile only waits on tiles with lower tickets of its own
// counter, which have already started: no deadlock.  G = 8 matches the round-robin
// dispatch of workgroups over the 8 XCDs, so a chain stays on one XCD's L2, and the blocked
// order makes the tiles an XCD runs together share their u and W panels there.
#include "gemm_core.h"
#include "kernels.h"

namespace rglru {

typedef GemmCfg<256, 128, 2, 4, false, 64, 2> CfgLru;
constexpr int kLruRows = CfgLru::BM;   // time steps per tile
constexpr int kLruCh = CfgLru::BC;     // channels per tile
constexpr int kTileBytes = kLruRows * kLruCh * 2;                  // one bf16 [rows x channels] tile
constexpr int kEpiScratch = (3 * kLruCh + 2 * kWindow * kLruCh) * 4;  // aggregates, carries, look-back
template <bool GATED>
constexpr int lru_lds_bytes() {
  return GATED ? 2 * kTileBytes + kEpiScratch : CfgLru::LDS_BYTES;
}
static_assert(kTileBytes + kEpiScratch <= CfgLru::LDS_BYTES, "epilogue LDS");
static_assert(2 * kTileBytes + kEpiScratch + 1024 <= 160 * 1024, "gated epilogue LDS");

int lru_chunks(int T) { return (T + kLruRows - 1) / kLruRows; }
long lru_tiles(int B, int T, int D) { return long(B) * ((D + kLruCh - 1) / kLruCh) * lru_chunks(T); }
size_t lru_status_bytes(int B, int T, int D) { return 3ull * lru_chunks(T) * size_t(B) * D * 4; }

static int lru_groups(int chains) {
  int g = 8;
  while (chains % g) g >>= 1;
  return g;
}

// The scan epilogue of lru_fused_kernel (see the file comment).  EDGE: the tile may have
// fewer than 256 valid rows or hold the sequence's final step.  GATED: multiply by p.gate.
template <bool EDGE, bool GATED>
__device__ __forceinline__ void lru_epilogue(const LruArgs& p, unsigned char* lds,
                                             f32x16_t (&acc)[CfgLru::MF][CfgLru::NF], int lane,
                                             int wave, int b, int tn, int tt, int t0, int rows) {
  typedef CfgLru C;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int B = p.B, T = p.T, D = p.D;
  const bf16_t* u = static_cast<const bf16_t*>(p.u);
  // LDS after the K loop: [0, 64 KB) the tile's u (then y) as 256 rows x 128 bf16 channels;
  // with a gate, [64 KB, 128 KB) its g tile; then per-channel aggregates, carries and the
  // look-back scratch.
  __syncthreads();   // every wave is done with the GEMM stages: the LDS is reused below
  bf16_t* tileU = reinterpret_cast<bf16_t*>(lds);
  float* eA = reinterpret_cast<float*>(lds + (GATED ? 2 : 1) * kTileBytes);
  float* eH = eA + kLruCh;
  float* eC = eH + kLruCh;
  float* eLb = eC + kLruCh;                          // look-back scratch, 2 kWindow per channel
  const int chv = min(kLruCh, D - tn * kLruCh);      // valid channels of the tile (64 or 128)
  const size_t rowbase = size_t(b) * T + t0;
  // A [256 rows x 128 channels] bf16 tile of src -> LDS [dst, dst + 64 KB), 16 bytes per
  // lane (4 rows of 256 B per wave instruction, kFetch instructions per wave); rows past the
  // sequence and chunks past D are clamped to valid addresses (their values are never used).
  constexpr int kFetch = kLruRows / 4 / C::NW;
  auto fetch_tile = [&](const bf16_t* src, int dst) {
    const bf16_t* sg = src + rowbase * D + tn * kLruCh;
#pragma unroll
    for (int it = 0; it < kFetch; ++it) {
      const int r = (it * C::NW + wave) * 4 + (lane >> 4);
      const int chunk = min(lane & 15, chv / 8 - 1);
      const bf16_t* gp = sg + size_t(min(r, rows - 1)) * D + chunk * 8;
      __builtin_amdgcn_global_load_lds((void*)gp, (void*)(lds + dst + (it * C::NW + wave) * 1024), 16, 0, 0);
    }
  };
  fetch_tile(u, 0);
  const int c = lane & 31, half = lane >> 5;
  const int chl = wn * 32 + c;                       // channel within the tile
  const int ch = tn * kLruCh + chl;
  const bool chok = chl < chv;
  const GateChan kc = gate_chan(p.ba[chok ? ch : tn * kLruCh], p.bx[chok ? ch : tn * kLruCh],
                                p.lam[chok ? ch : tn * kLruCh], p.c);
  if (GATED) {
    fetch_tile(static_cast<const bf16_t*>(p.gate), kTileBytes);
    wait_dma_barrier<kFetch>();                      // the u tile is in LDS (g may still land)
  } else {
    wait_dma_barrier<0>();                           // the u tile is in LDS
  }
  // Group q = 4 mf + gq of this lane covers tile rows wm*128 + 32 mf + 8 gq + 4 half + rr,
  // rr = 0..3 (consecutive time steps); tb[(32 mf + 8 gq + rr) * kLruCh] is the LDS element
  // of row rr (constant offsets).  The first pass turns the accumulator pair (z^a, z^x) of
  // each element into (a_t, beta_t u_t) in place, so the second pass finds them there.
  bf16_t* tb = tileU + (wm * C::WTM + 4 * half) * kLruCh + chl;
  // rows of this lane's groups are lrow0 + 32 mf + 8 gq + rr; those >= lim are past the end
  const int lrow0 = wm * C::WTM + 4 * half;
  const int lim = rows - lrow0;
  // Per group: the summary (A = prod a, H) and the running composition over the 32 groups
  // of the wave's 128 rows in time order (for each gq the lower-half lane's group comes
  // first, then the upper-half lane's).  pre[q] is the map in front of this lane's group q.
  float preA[16], preH[16];
  float RA = 1.f, RH = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    float Aq = 1.f, Hq = 0.f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int mf = q >> 2, gq = q & 3, v = gq * 4 + rr;
      const int rel = mf * 32 + 8 * gq + rr;
      float a, beta;
      gate_fast(acc[mf][0][v], acc[mf][1][v], kc, a, beta);
      const float uv = bf2f(tb[rel * kLruCh]);      // rows past the end hold clamped copies
      const bool ok = !EDGE || rel < lim;
      a = ok ? a : 1.f;
      const float bu = ok ? beta * uv : 0.f;
      acc[mf][0][v] = a;
      acc[mf][1][v] = bu;
      Hq = fmaf(a, Hq, bu);
      Aq = Aq * a;
    }
    const WaveHalves sa = wave_halves(Aq), sh = wave_halves(Hq);
    const float A0 = sa.lo, H0 = sh.lo;   // rows 8gq .. 8gq+3 (the lower-half lane's group)
    const float A1 = sa.hi, H1 = sh.hi;   // rows 8gq+4 .. 8gq+7
    const float R0A = RA, R0H = RH;
    RH = fmaf(A0, RH, H0);
    RA = A0 * RA;
    preA[q] = half ? RA : R0A;
    preH[q] = half ? RH : R0H;
    RH = fmaf(A1, RH, H1);
    RA = A1 * RA;
    __builtin_amdgcn_sched_barrier(0);   // one group at a time: bounds the live registers
  }
  if (wm == 0 && half == 0) { eA[chl] = RA; eH[chl] = RH; }
  __syncthreads();                                   // also: every wave is done reading u
  float A0w = 1.f, H0w = 0.f;
  if (wm == 1) { A0w = eA[chl]; H0w = eH[chl]; }
  if (wm == 1 && half == 0) {
    // tile aggregate: the upper 128 rows, then the lower 128
    const float At = RA * A0w, Ht = fmaf(RA, H0w, RH);
    float carry = 0.f;
    if (chok) {
      const int nchunks = (T + kLruRows - 1) / kLruRows;
      const size_t BD = size_t(B) * D, base = size_t(b) * D + ch;
      uint32_t* incl = p.status;
      uint32_t* aggA = incl + size_t(nchunks) * BD;
      uint32_t* aggH = aggA + size_t(nchunks) * BD;
      if (tt > 0) {
        publish<float>(aggA + size_t(tt) * BD + base, At);
        publish<float>(aggH + size_t(tt) * BD + base, Ht);
        carry = lookback_carry<float>(incl + base, aggA + base, aggH + base, tt, BD,
                                      eLb + chl * 2 * kWindow, eLb + chl * 2 * kWindow + kWindow,
                                      p.max_polls, p.stall);
      } else {
        carry = p.h0 ? p.h0[base] : 0.f;
      }
      publish<float>(incl + size_t(tt) * BD + base, fmaf(At, carry, Ht));
    }
    eC[chl] = carry;
  }
  if (GATED) wait_dma_barrier<0>();                  // the g tile is in LDS too
  else __syncthreads();
  const float carry = eC[chl];
  const float hin = wm == 0 ? carry : fmaf(A0w, carry, H0w);
  const int lastrel = T - 1 - t0 - lrow0;            // the final step, if in this lane's rows
  float hlast = 0.f;
  bool haslast = false;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    float h = fmaf(preA[q], hin, preH[q]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      h = fmaf(acc[q >> 2][0][(q & 3) * 4 + rr], h, acc[q >> 2][1][(q & 3) * 4 + rr]);
      const int rel = (q >> 2) * 32 + 8 * (q & 3) + rr;
      const float o = GATED ? h * bf2f(tb[kTileBytes / 2 + rel * kLruCh]) : h;
      tb[rel * kLruCh] = f2bf(o);
      if (EDGE) {
        hlast = rel == lastrel ? h : hlast;
        haslast = haslast || rel == lastrel;
      }
    }
  }
  if (EDGE && haslast && chok && p.hT) p.hT[size_t(b) * D + ch] = hlast;
  __syncthreads();
  // y rows of the tile -> HBM, 16 bytes per lane
  bf16_t* yg = static_cast<bf16_t*>(p.y) + rowbase * D + tn * kLruCh;
#pragma unroll
  for (int it = 0; it < kLruRows / 4 / C::NW; ++it) {
    const int r = (it * C::NW + wave) * 4 + (lane >> 4);
    const int chunk = lane & 15;
    if ((!EDGE || r < rows) && chunk * 8 < chv)
      *reinterpret_cast<uint4*>(yg + size_t(r) * D + chunk * 8) =
          *reinterpret_cast<const uint4*>(tileU + r * kLruCh + chunk * 8);
  }
}

template <bool GATED>
__global__ __launch_bounds__(CfgLru::NW * 64, 2) void lru_fused_kernel(LruArgs p) {
  typedef CfgLru C;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[lru_lds_bytes<GATED>()];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ uint32_t s_ticket;
  const int G = p.groups, g = blockIdx.x % G;
  const int B = p.B, T = p.T, D = p.D;
  const int NT = (D + kLruCh - 1) / kLruCh;
  const int per_level = B * NT / G;
  const int bw = p.chain_bw;
  auto tile_of = [&](int k, int& b, int& tn, int& tt) {
    tt = k / per_level;
    // position of the chain in the blocked chain order (blocks of bw sequences, channel
    // tile by channel tile): group g owns positions g * per_level .. + per_level - 1
    const int o = g * per_level + k % per_level;
    const int blk = o / (bw * NT), rem = o % (bw * NT);
    b = blk * bw + rem % bw;
    tn = rem / bw;
  };
  auto operands = [&](int b, int tn, int tt) {
    TileOperands op;
    op.A = static_cast<const bf16_t*>(p.u); op.A2 = nullptr;
    op.B0 = static_cast<const bf16_t*>(p.Wa);
    op.B1 = static_cast<const bf16_t*>(p.Wx);
    op.lda = D; op.ldb = D; op.K = D;
    op.a_row0 = b * T + tt * kLruRows; op.a_rows = min(kLruRows, T - tt * kLruRows);
    op.b_row0 = tn * kLruCh; op.b_rows = min(kLruCh, D - tn * kLruCh);
    return op;
  };
  // The ticket's atomic round trip overlaps the first k-step's operand loads: those are
  // issued for the tile this workgroup gets when the tickets of its group go in launch
  // order (ticket blockIdx / G); if the ticket says otherwise, the loads are waited for and
  // the tile's own are issued instead.
  uint32_t ticket = 0;
  if (tid == 0) ticket = atomicAdd(p.counters + g, 1u);
  int b, tn, tt;
  const int kp = (int(blockIdx.x) / G + p.ticket_guess) % (int(gridDim.x) / G);
  tile_of(kp, b, tn, tt);
  TileOperands op = operands(b, tn, tt);
  GemmDma<C, false>(op, lane, wave).issue(op, lds, wave, 0);
  if (tid == 0) s_ticket = ticket;  // after the loads are issued: the wait for the atomic
                                    // (vmcnt in issue order) leaves them in flight
  wait_dma_barrier<C::QPW>();       // the ticket is in LDS; the first k-step may still land
  const int k = __builtin_amdgcn_readfirstlane(int(s_ticket));
  const bool hit = k == kp;
  if (!hit) {
    wait_dma_barrier<0>();          // every wave's loads into stage 0 have landed
    tile_of(k, b, tn, tt);
    op = operands(b, tn, tt);
  }
  const int t0 = tt * kLruRows;
  const int rows = min(kLruRows, T - t0);
  f32x16_t acc[C::MF][C::NF];
  gemm_mainloop<C, false>(op, lds, lane, wave, acc, hit);

  // ---------------------------------------------------------------- scan epilogue
  lru_epilogue<true, GATED>(p, lds, acc, lane, wave, b, tn, tt, t0, rows);
}

hipError_t launch_lru_fused(const LruArgs& a_in, bool prefilled, hipStream_t s) {
  LruArgs a = a_in;
  if (a.ticket_guess < 0) a.ticket_guess = 0;
  const int NT = (a.D + kLruCh - 1) / kLruCh;
  const int chains = a.B * NT;
  a.groups = lru_groups(chains);
  // a group's chains span bw sequences (u panels) and about per_level / bw channel tiles
  // (W panels) per time level; blocks of up to 4 sequences keep both few: at 8 x 2048 x 2560,
  // 4 u panels and 5 W panels per level instead of 8 and 3 (the kernel's fetches beyond L2,
  // FETCH_SIZE, drop from 1.04 to 0.83 GB per launch at the same speed)
  a.chain_bw = a.B % 4 == 0 ? 4 : (a.B % 2 == 0 ? 2 : 1);
  if (!prefilled) {
    const hipError_t e = launch_fill_status(a.status, lru_status_bytes(a.B, a.T, a.D) / 4,
                                            a.counters, kCounterWords, s);
    if (e != hipSuccess) return e;
  }
  const int tiles = chains * lru_chunks(a.T);
  if (a.gate) lru_fused_kernel<true><<<tiles, CfgLru::NW * 64, 0, s>>>(a);
  else lru_fused_kernel<false><<<tiles, CfgLru::NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rglru
