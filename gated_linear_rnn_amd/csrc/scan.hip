// Diagonal linear scan of the RG-LRU, Eq. (4) of the Griffin model-architecture page
// ("Real-Gated Linear Recurrent Unit (RG-LRU)" section):
//     h_t = a_t h_{t-1} + beta_t u_t,   beta_t = sqrt(1 - a_t^2) i_t,   y_t = h_t,
// evaluated as a chunked parallel scan (the blog page "Griffin's Compromise", "Term
// explanation: Parallel scan": chunk subtotals computed in parallel, each chunk's summary
// passed on to the next).  Every step is elementwise over channels and the kernel moves
// 12 bytes per element at bf16 I/O (x 2, a 4, beta 4, y 2), so it is HBM-bound.
//
// Work decomposition (one workgroup = 256 threads = one tile of 128 time steps x 64
// channels of one sequence):
//   * thread (tg, cg): time group tg in [0,16) owns 8 consecutive steps, channel group cg
//     in [0,16) owns 4 consecutive channels, so a wave's loads of a and beta cover four
//     256-byte channel-contiguous row segments;
//   * x rows t0-3 .. t0+127 are staged through LDS with coalesced loads and the width-4
//     conv (the "Recurrent block" Conv1D) is recomputed from them with the same fma order
//     as the stand-alone conv, so u is bit-identical to the u the gate projection used;
//   * each thread scans its 8 steps from zero to the affine summary (A = prod a, H), the
//     16 time-group summaries are combined in LDS, and the tile summary is chained across
//     tiles with a decoupled look-back (tiles take tickets in time order from an atomic
//     counter, so every tile a tile waits on has already started: no deadlock);
//   * each thread then re-runs its 8 steps from its exact incoming state and writes y.
// The scan state type Acc is fp32 for bf16 I/O and fp64 for fp32 I/O.
#include "rglru_device.h"
#include "kernels.h"

namespace rglru {

constexpr int kSteps = 8;                 // steps per thread
constexpr int kTG = 16;                   // time groups per tile
constexpr int kChunk = kSteps * kTG;      // 128 time steps per tile
constexpr int kCh = 64;                   // channels per tile

int scan_chunks(int T) { return (T + kChunk - 1) / kChunk; }
size_t scan_status_bytes(int B, int T, int D, int acc_bytes) {
  return 3ull * scan_chunks(T) * size_t(B) * D * size_t(acc_bytes);
}

// Compose the summaries of time groups [q0, q1) of this tile (ascending order of
// application) for 4 channels: h -> A h + H.
template <typename Acc>
__device__ __forceinline__ void compose_groups(const Acc (*sA)[kCh], const Acc (*sH)[kCh], int c0,
                                               int q0, int q1, int step, Acc* A, Acc* H) {
#pragma unroll
  for (int j = 0; j < 4; ++j) { A[j] = Acc(1); H[j] = Acc(0); }
  for (int q = q0; q != q1; q += step)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const Acc Aq = sA[q][c0 + j], Hq = sH[q][c0 + j];
      H[j] = fmaA(Aq, H[j], Hq);
      A[j] = Aq * A[j];
    }
}

template <typename IO, typename Acc>
__global__ __launch_bounds__(256) void scan_fwd_kernel(ScanFwdArgs p) {
  typedef typename Words<Acc>::W W;
  __shared__ uint32_t s_ticket;
  __shared__ float xs[(kChunk + 3) * kCh];
  __shared__ Acc sA[kTG][kCh], sH[kTG][kCh];
  __shared__ Acc sCarry[kCh];
  __shared__ Acc sLb[16][2][kWindow];

  const int B = p.B, T = p.T, D = p.D;
  const int tid = threadIdx.x;
  if (tid == 0) s_ticket = atomicAdd(p.counter, 1u);
  __syncthreads();
  const int nblk = B * (D / kCh);
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int tk = int(s_ticket);
  const int chunk = tk / nblk, blk = tk % nblk;
  const int b = blk / (D / kCh), d0 = (blk % (D / kCh)) * kCh;
  const int t0 = chunk * kChunk;
  const int cg = tid & 15, tg = tid >> 4;
  const int d = d0 + 4 * cg;
  const size_t BD = size_t(B) * D;

  // gates for this thread's steps (issued first: the longest-latency loads)
  float4 ga[kSteps], gb[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int t = t0 + tg * kSteps + s;
    if (t < T) {
      const size_t o = (size_t(b) * T + t) * D + d;
      ga[s] = *reinterpret_cast<const float4*>(p.a + o);
      gb[s] = *reinterpret_cast<const float4*>(p.beta + o);
    } else {
      ga[s] = p.from_ri ? make_float4(0, 0, 0, 0) : make_float4(1, 1, 1, 1);
      gb[s] = make_float4(0, 0, 0, 0);
    }
  }
  // stage x rows t0-3 .. t0+kChunk-1 (fp32 in LDS)
  const IO* x = static_cast<const IO*>(p.x);
  const IO* cs = static_cast<const IO*>(p.conv_state);
  for (int idx = tid; idx < (kChunk + 3) * 16; idx += 256) {
    const int rr = idx >> 4, q = idx & 15;
    const int t = t0 - 3 + rr;
    float4 v = make_float4(0, 0, 0, 0);
    if (t >= 0 && t < T) v = Io<IO>::load4(x + (size_t(b) * T + t) * D + d0 + 4 * q);
    else if (t < 0 && cs) v = Io<IO>::load4(cs + (size_t(b) * 3 + 3 + t) * D + d0 + 4 * q);
    *reinterpret_cast<float4*>(&xs[rr * kCh + 4 * q]) = v;
  }
  float4 w0 = make_float4(0, 0, 0, 0), w1 = w0, w2 = w0, w3 = w0, cb = w0, Lv = w0;
  const bool conv = p.conv_w != nullptr;
  if (conv) {
    const IO* w = static_cast<const IO*>(p.conv_w);
    w0 = Io<IO>::load4(w + d); w1 = Io<IO>::load4(w + D + d);
    w2 = Io<IO>::load4(w + 2 * D + d); w3 = Io<IO>::load4(w + 3 * D + d);
    if (p.conv_b) cb = *reinterpret_cast<const float4*>(p.conv_b + d);
  }
  if (p.from_ri) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f4set(Lv, j, log_sigmoidf(p.lam[d + j]));
  }
  __syncthreads();

  // a_t and beta_t u_t for each step
  Acc av[kSteps][4], bu[kSteps][4];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int rr = tg * kSteps + s + 3;
    const float4 x0 = *reinterpret_cast<const float4*>(&xs[rr * kCh + 4 * cg]);
    float4 u = x0;
    if (conv) {
      const float4 x1 = *reinterpret_cast<const float4*>(&xs[(rr - 1) * kCh + 4 * cg]);
      const float4 x2 = *reinterpret_cast<const float4*>(&xs[(rr - 2) * kCh + 4 * cg]);
      const float4 x3 = *reinterpret_cast<const float4*>(&xs[(rr - 3) * kCh + 4 * cg]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f4set(u, j, conv_u<IO>(f4get(cb, j), f4get(w0, j), f4get(w1, j), f4get(w2, j),
                               f4get(w3, j), f4get(x0, j), f4get(x1, j), f4get(x2, j),
                               f4get(x3, j)));
    }
    const bool valid = t0 + tg * kSteps + s < T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = f4get(ga[s], j), beta = f4get(gb[s], j);
      if (p.from_ri) {
        const Gate g = gate_from_ri(a, beta, f4get(Lv, j), p.c);
        a = valid ? g.a : 1.f;
        beta = valid ? g.m * g.i : 0.f;
      }
      av[s][j] = Acc(a);
      bu[s][j] = Acc(beta) * Acc(f4get(u, j));
    }
  }

  // local summary of this thread's steps: h -> A h + H
  Acc A[4], H[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { A[j] = Acc(1); H[j] = Acc(0); }
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      H[j] = fmaA(av[s][j], H[j], bu[s][j]);
      A[j] = A[j] * av[s][j];
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) { sA[tg][4 * cg + j] = A[j]; sH[tg][4 * cg + j] = H[j]; }
  __syncthreads();

  if (tg == 0) {
    // tile aggregate, publish, look back, publish the inclusive state
    Acc Ag[4], Hg[4];
    compose_groups<Acc>(sA, sH, 4 * cg, 0, kTG, 1, Ag, Hg);
    W* incl = static_cast<W*>(p.status);
    W* aggA = incl + size_t(nchunks) * BD;
    W* aggH = aggA + size_t(nchunks) * BD;
    const size_t base = size_t(b) * D + d;
    if (chunk > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        publish<Acc>(aggA + size_t(chunk) * BD + base + j, Ag[j]);
        publish<Acc>(aggH + size_t(chunk) * BD + base + j, Hg[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Acc carry;
      if (chunk == 0) carry = p.h0 ? Acc(p.h0[base + j]) : Acc(0);
      else carry = lookback_carry<Acc>(incl + base + j, aggA + base + j, aggH + base + j, chunk,
                                       BD, sLb[cg][0], sLb[cg][1]);
      publish<Acc>(incl + size_t(chunk) * BD + base + j, fmaA(Ag[j], carry, Hg[j]));
      sCarry[4 * cg + j] = carry;
    }
  }
  // exclusive prefix of the time groups before this one
  Acc Ap[4], Hp[4];
  compose_groups<Acc>(sA, sH, 4 * cg, 0, tg, 1, Ap, Hp);
  __syncthreads();

  Acc h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = fmaA(Ap[j], sCarry[4 * cg + j], Hp[j]);
  IO* y = static_cast<IO*>(p.y);
  Acc* h_all = static_cast<Acc*>(p.h_all);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int t = t0 + tg * kSteps + s;
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = fmaA(av[s][j], h[j], bu[s][j]);
    if (t < T) {
      const size_t o = (size_t(b) * T + t) * D + d;
      const float4 hf = make_float4(float(h[0]), float(h[1]), float(h[2]), float(h[3]));
      if (y) Io<IO>::store4(y + o, hf);
      if (h_all) {
#pragma unroll
        for (int j = 0; j < 4; ++j) h_all[o + j] = h[j];
      }
      if (t == T - 1 && p.h_T) *reinterpret_cast<float4*>(p.h_T + size_t(b) * D + d) = hf;
    }
  }
}

template <typename IO, typename Acc>
hipError_t launch_scan_fwd(const ScanFwdArgs& a, hipStream_t s) {
  if (!a.prefilled) {
    const hipError_t e = launch_fill_status(static_cast<uint32_t*>(a.status),
                                            scan_status_bytes(a.B, a.T, a.D, sizeof(Acc)) / 4, a.counter, 1, s);
    if (e != hipSuccess) return e;
  }
  const int tiles = scan_chunks(a.T) * a.B * (a.D / kCh);
  scan_fwd_kernel<IO, Acc><<<tiles, 256, 0, s>>>(a);
  return hipGetLastError();
}
template hipError_t launch_scan_fwd<float, double>(const ScanFwdArgs&, hipStream_t);
template hipError_t launch_scan_fwd<bf16_t, float>(const ScanFwdArgs&, hipStream_t);

// ------------------------------------------------------------------ reverse scan
// Backward through Eq. (4) (the pages give no backward; chain rule).  With G_t the total
// derivative of h_t and g_t = a_t G_t the part handed to step t-1:
//     G_t = dy_t + g_{t+1},   g_t = a_t (dy_t + g_{t+1}),   g_T = dh_T,   dh0 = g_0,
// the same affine recurrence run backwards in time, chunked and chained exactly like the
// forward (tiles take tickets from the last time chunk to the first).  Per element it
// then forms the local gradients:
//     d(log a) = G (a h_{t-1} - (a^2/m) i u)   [m-path term 0 where m = 0]
//     dz^a = c L d(log a) r (1-r),  dz^x = G m u i (1-i),  du_direct = G m i,
// and per-tile fp64 partial sums of dz^a, dz^x and c r d(log a) (for db_a, db_x, dLambda).
template <typename IO, typename Acc>
__global__ __launch_bounds__(256) void scan_bwd_kernel(ScanBwdArgs p) {
  typedef typename Words<Acc>::W W;
  __shared__ uint32_t s_ticket;
  __shared__ Acc sA[kTG][kCh], sH[kTG][kCh];
  __shared__ Acc sCarry[kCh];
  __shared__ Acc sLb[16][2][kWindow];
  __shared__ double sRed[kTG][3][kCh];

  const int B = p.B, T = p.T, D = p.D;
  const int tid = threadIdx.x;
  if (tid == 0) s_ticket = atomicAdd(p.counter, 1u);
  __syncthreads();
  const int nblk = B * (D / kCh);
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int tk = int(s_ticket);
  const int pos = tk / nblk, blk = tk % nblk;       // chain position 0 = last time chunk
  const int chunk = nchunks - 1 - pos;
  const int b = blk / (D / kCh), d0 = (blk % (D / kCh)) * kCh;
  const int t0 = chunk * kChunk;
  const int cg = tid & 15, tg = tid >> 4;
  const int d = d0 + 4 * cg;
  const size_t BD = size_t(B) * D;

  // Inputs stream through registers one step at a time (the next step's loads are in
  // flight while the current one is computed), which keeps the kernel near 128 VGPRs so
  // that four workgroups share a CU.
  const IO* u = static_cast<const IO*>(p.u);
  const IO* dy = static_cast<const IO*>(p.dy);
  const Acc* h_all = static_cast<const Acc*>(p.h_all);
  float4 Lv;
#pragma unroll
  for (int j = 0; j < 4; ++j) f4set(Lv, j, log_sigmoidf(p.lam[d + j]));
  auto row_of = [&](int s) { return size_t(b) * T + (t0 + tg * kSteps + s); };
  auto valid = [&](int s) { return t0 + tg * kSteps + s < T; };
  // a_t of 4 channels from r_t (identity a = 1 on padded steps)
  auto gate_a = [&](const float4& r, bool ok, int j) {
    return ok ? gate_from_ri(f4get(r, j), 0.f, f4get(Lv, j), p.c).a : 1.f;
  };

  // pass 1: local summary, backwards over this thread's steps: g -> A g + H
  Acc A[4], H[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { A[j] = Acc(1); H[j] = Acc(0); }
  {
    float4 rn = make_float4(0, 0, 0, 0), dn = rn;
    if (valid(kSteps - 1)) {
      rn = *reinterpret_cast<const float4*>(p.r + row_of(kSteps - 1) * D + d);
      dn = Io<IO>::load4(dy + row_of(kSteps - 1) * D + d);
    }
#pragma unroll 1
    for (int s = kSteps - 1; s >= 0; --s) {
      const float4 rc = rn, dc = dn;
      const bool ok = valid(s);
      if (s > 0 && valid(s - 1)) {
        rn = *reinterpret_cast<const float4*>(p.r + row_of(s - 1) * D + d);
        dn = Io<IO>::load4(dy + row_of(s - 1) * D + d);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const Acc a = gate_a(rc, ok, j);
        H[j] = a * (Acc(f4get(dc, j)) + H[j]);
        A[j] = A[j] * a;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) { sA[tg][4 * cg + j] = A[j]; sH[tg][4 * cg + j] = H[j]; }
  __syncthreads();

  if (tg == 0) {
    Acc Ag[4], Hg[4];
    compose_groups<Acc>(sA, sH, 4 * cg, kTG - 1, -1, -1, Ag, Hg);
    W* incl = static_cast<W*>(p.status);
    W* aggA = incl + size_t(nchunks) * BD;
    W* aggH = aggA + size_t(nchunks) * BD;
    const size_t base = size_t(b) * D + d;
    if (pos > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        publish<Acc>(aggA + size_t(pos) * BD + base + j, Ag[j]);
        publish<Acc>(aggH + size_t(pos) * BD + base + j, Hg[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Acc carry;
      if (pos == 0) carry = p.dh_T ? Acc(p.dh_T[base + j]) : Acc(0);
      else carry = lookback_carry<Acc>(incl + base + j, aggA + base + j, aggH + base + j, pos, BD,
                                       sLb[cg][0], sLb[cg][1]);
      publish<Acc>(incl + size_t(pos) * BD + base + j, fmaA(Ag[j], carry, Hg[j]));
      sCarry[4 * cg + j] = carry;
    }
  }
  Acc Ap[4], Hp[4];
  compose_groups<Acc>(sA, sH, 4 * cg, kTG - 1, tg, -1, Ap, Hp);
  __syncthreads();

  // pass 2: the local gradients, backwards from the exact incoming g
  Acc g[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) g[j] = fmaA(Ap[j], sCarry[4 * cg + j], Hp[j]);
  double sdza[4] = {0, 0, 0, 0}, sdzi[4] = {0, 0, 0, 0}, sdl[4] = {0, 0, 0, 0};
  const size_t ld2 = size_t(2) * D;
  const Acc cL[4] = {Acc(p.c) * Acc(f4get(Lv, 0)), Acc(p.c) * Acc(f4get(Lv, 1)),
                     Acc(p.c) * Acc(f4get(Lv, 2)), Acc(p.c) * Acc(f4get(Lv, 3))};
  struct StepIn {
    float4 r, i, u, dy;
    Acc hp[4];
  };
  auto load_step = [&](int s, StepIn& in) {
    const int t = t0 + tg * kSteps + s;
    if (t < T) {
      const size_t o = (size_t(b) * T + t) * D + d;
      in.r = *reinterpret_cast<const float4*>(p.r + o);
      in.i = *reinterpret_cast<const float4*>(p.i + o);
      in.u = Io<IO>::load4(u + o);
      in.dy = Io<IO>::load4(dy + o);
      if (t > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) in.hp[j] = h_all[o - D + j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) in.hp[j] = p.h0 ? Acc(p.h0[size_t(b) * D + d + j]) : Acc(0);
      }
    } else {
      in.r = in.i = in.u = in.dy = make_float4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) in.hp[j] = Acc(0);
    }
  };
  StepIn cur, nxt;
  load_step(kSteps - 1, nxt);
#pragma unroll 1
  for (int s = kSteps - 1; s >= 0; --s) {
    cur = nxt;
    if (s > 0) load_step(s - 1, nxt);
    const int t = t0 + tg * kSteps + s;
    const bool ok = t < T;
    float4 dza, dzi, dud;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const Gate gt = gate_from_ri(f4get(cur.r, j), f4get(cur.i, j), f4get(Lv, j), p.c);
      const Acc a = ok ? gt.a : 1.f, m = ok ? gt.m : 0.f;
      const Acc r = f4get(cur.r, j), ii = f4get(cur.i, j), uv = f4get(cur.u, j);
      const Acc G = Acc(f4get(cur.dy, j)) + g[j];
      const Acc mterm = m > Acc(0) ? ((a * a) / m) * ii * uv : Acc(0);
      const Acc dl = G * (a * cur.hp[j] - mterm);
      const Acc zr = cL[j] * dl * r * (Acc(1) - r);
      const Acc zi = (G * m * uv) * ii * (Acc(1) - ii);
      f4set(dza, j, float(zr));
      f4set(dzi, j, float(zi));
      f4set(dud, j, float(G * m * ii));
      if (ok) {
        sdza[j] += double(zr);
        sdzi[j] += double(zi);
        sdl[j] += double(Acc(p.c) * r * dl);
      }
      g[j] = a * G;
    }
    if (ok) {
      const size_t row = size_t(b) * T + t;
      *reinterpret_cast<float4*>(p.du + row * D + d) = dud;
      if (sizeof(IO) == 2) {
        float4 lo_a, lo_i;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f4set(lo_a, j, f4get(dza, j) - Io<bf16_t>::round(f4get(dza, j)));
          f4set(lo_i, j, f4get(dzi, j) - Io<bf16_t>::round(f4get(dzi, j)));
        }
        bf16_t* hi = static_cast<bf16_t*>(p.dz_hi);
        bf16_t* lo = static_cast<bf16_t*>(p.dz_lo);
        Io<bf16_t>::store4(hi + row * ld2 + d, dza);
        Io<bf16_t>::store4(hi + row * ld2 + D + d, dzi);
        Io<bf16_t>::store4(lo + row * ld2 + d, lo_a);
        Io<bf16_t>::store4(lo + row * ld2 + D + d, lo_i);
      } else {
        float* z = static_cast<float*>(p.dz_hi);
        *reinterpret_cast<float4*>(z + row * ld2 + d) = dza;
        *reinterpret_cast<float4*>(z + row * ld2 + D + d) = dzi;
      }
      if (t == 0 && p.dh0)
        *reinterpret_cast<float4*>(p.dh0 + size_t(b) * D + d) =
            make_float4(float(g[0]), float(g[1]), float(g[2]), float(g[3]));
    }
  }
  // fixed-order per-tile partial sums
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sRed[tg][0][4 * cg + j] = sdza[j];
    sRed[tg][1][4 * cg + j] = sdzi[j];
    sRed[tg][2][4 * cg + j] = sdl[j];
  }
  __syncthreads();
  if (tid < 3 * kCh) {
    const int qn = tid / kCh, c = tid % kCh;
    double acc = 0.0;
    for (int q = 0; q < kTG; ++q) acc += sRed[q][qn][c];
    p.partial[(size_t(b) * nchunks + chunk) * 3 * D + size_t(qn) * D + d0 + c] = acc;
  }
}

template <typename IO, typename Acc>
hipError_t launch_scan_bwd(const ScanBwdArgs& a, hipStream_t s) {
  const hipError_t e = launch_fill_status(static_cast<uint32_t*>(a.status),
                                          scan_status_bytes(a.B, a.T, a.D, sizeof(Acc)) / 4, a.counter, 1, s);
  if (e != hipSuccess) return e;
  const int tiles = scan_chunks(a.T) * a.B * (a.D / kCh);
  scan_bwd_kernel<IO, Acc><<<tiles, 256, 0, s>>>(a);
  return hipGetLastError();
}
template hipError_t launch_scan_bwd<float, double>(const ScanBwdArgs&, hipStream_t);
template hipError_t launch_scan_bwd<bf16_t, float>(const ScanBwdArgs&, hipStream_t);

}  // namespace rglru
