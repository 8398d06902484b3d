// Diagonal linear scan of the RG-LRU, Eq. (4) of the Griffin model-architecture page
// ("Real-Gated Linear Recurrent Unit (RG-LRU)" section):
//     h_t = a_t h_{t-1} + beta_t u_t,   beta_t = sqrt(1 - a_t^2) i_t,   y_t = h_t,
// evaluated as a chunked parallel scan (the blog page "Griffin's Compromise", "Term
// explanation: Parallel scan": chunk subtotals computed in parallel, each chunk's summary
// passed on to the next).  Every step is elementwise over channels and the forward moves
// 12 bytes per element at bf16 I/O (x 2, a 4, beta 4, y 2), so it is HBM-bound: the
// design goal is to keep enough loads in flight on every CU.
//
// Forward work decomposition (one workgroup = 256 threads = one tile of 64 time steps x
// 64 channels of one sequence):
//   * thread (tg, cg): time group tg in [0,16) owns 4 consecutive steps, channel group cg
//     in [0,16) owns 4 consecutive channels, so one wave load instruction covers four
//     256-byte channel-contiguous row segments of a or beta;
//   * every load of the tile is issued up front, straight into registers: a and beta of
//     the thread's 4 steps and the x rows t-3 .. t+3 around them, from which the width-4
//     conv (the "Recurrent block" Conv1D) is recomputed with the same fma order as the
//     stand-alone conv, so u is bit-identical to the u the gate projection used (the conv
//     weights of the tile's channels pass through LDS).  At most 128 VGPRs at bf16 I/O:
//     four workgroups share a CU, so while one waits on its predecessor or writes y, the
//     others' loads are in flight;
//   * the gates arrive as (a_t, beta_t), as (r_t, i_t), or (fp32 I/O) as the raw
//     projections W_a u_t and W_x u_t; in the last two forms the tile evaluates Eq. (2)-(4)
//     itself, in fp64 for the fp64 state;
//   * each thread scans its 4 steps from zero to the affine summary (A = prod a, H), the
//     16 time-group summaries are combined in LDS, and the tile summary is chained across
//     tiles with a decoupled look-back, one lane per channel so that the 64 channels' polls
//     overlap;
//   * each thread then re-runs its 4 steps from its exact incoming state and writes y.
// Tiles of a chain (sequence b, channel block) are numbered time level by time level
// within the chain's group g = blockIdx mod G (group g owns the chains g, g + G, ...), so
// a tile's predecessors always have lower indices and normally started earlier.  No ticket
// counter is taken: its atomic round trip, paid before any load could be issued, cost
// about a third of the kernel's time.  Safety does not rest on the dispatch order either:
// a look-back that finds a predecessor unpublished for long computes that chunk's summary
// itself from memory, bit for bit what the predecessor would publish.
// The scan state type Acc is fp32 for bf16 I/O and fp64 for fp32 I/O.  The reverse scan
// of the backward (below) keeps 128-step tiles.
#include "rglru_device.h"
#include "kernels.h"

namespace rglru {

constexpr int kSteps = 8;                 // reverse scan: steps per thread
constexpr int kTG = 16;                   // time groups per tile (both directions)
constexpr int kChunk = kSteps * kTG;      // reverse scan: 128 time steps per tile
constexpr int kCh = 64;                   // channels per tile
constexpr int kFSteps = 4;                // forward: steps per thread
constexpr int kFChunk = kFSteps * kTG;    // forward: 64 time steps per tile

int scan_chunks(int T) { return (T + kChunk - 1) / kChunk; }
__host__ __device__ inline int scan_fwd_chunks(int T) { return (T + kFChunk - 1) / kFChunk; }
long scan_fwd_tiles(int B, int T, int D) { return long(B) * (D / kCh) * scan_fwd_chunks(T); }

// The gates-from-projections mode exists for the fp64 scan state (fp32 I/O) only; the
// fp32-state instantiation compiles it out.
template <typename Acc>
__device__ __forceinline__ bool from_z_mode(const ScanFwdArgs& p) {
  return sizeof(Acc) == 8 && p.from_z;
}

// Sized for the finer forward chunking (the backward runs both scans on one buffer).
size_t scan_status_bytes(int B, int T, int D, int acc_bytes) {
  const int ch = scan_fwd_chunks(T) > scan_chunks(T) ? scan_fwd_chunks(T) : scan_chunks(T);
  return 3ull * ch * size_t(B) * D * size_t(acc_bytes);
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

// 4 consecutive I/O elements kept in their storage format until used.
template <typename IO> struct Raw4;
template <> struct Raw4<bf16_t> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint2(0u, 0u); }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t w = j < 2 ? v.x : v.y;
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Raw4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ float get(int j) const { return f4get(v, j); }
};

// Tile groups: the largest of 8, 4, 2, 1 dividing the number of chains.
static int scan_groups(int chains) {
  int g = 8;
  while (chains % g) g >>= 1;
  return g;
}

// (a_t, beta_t u_t) of one element: the identity map past the end of the sequence, the gates
// recomputed from (r, i) when the inputs are those.  Shared by the tile pass and the direct
// chunk summary below, so both produce the same bits.  With an fp64 state (fp32 I/O) the
// recomputed a_t and m_t are fp64 too: an fp32 a_t would carry the small rounding bias of
// the fp32 exponential into the recurrence, where it compounds over the steps.
template <typename Acc>
__device__ __forceinline__ void scan_elem(bool valid, float ga, float gb, float u, float L,
                                          bool from_ri, bool from_z, float zba, float zbx,
                                          float c, Acc& av, Acc& bu) {
  if (sizeof(Acc) == 8 && valid && (from_ri || from_z)) {
    const float r = from_z ? sigmoidf_stable(ga + zba) : ga;
    const float i = from_z ? sigmoidf_stable(gb + zbx) : gb;
    const GateAmD g = gate_am(r, double(L), c);
    av = Acc(g.a);
    bu = Acc(g.m * double(i)) * Acc(u);
    return;
  }
  // (the projections mode exists for the fp64 state only: see from_z_mode)
  float a = 1.f, beta = 0.f;
  if (valid) {
    a = ga;
    beta = gb;
    if (from_ri) {
      const Gate g = gate_from_ri(a, beta, L, c);
      a = g.a;
      beta = g.m * g.i;
    }
  }
  av = Acc(a);
  bu = valid ? Acc(beta) * Acc(u) : Acc(0);
}

// Summary (A, H) of one channel over forward chunk `chunk`, read straight from memory and
// composed in exactly the order of the tile pass (4-step groups folded from (1, 0), then
// the 16 groups in time order), so it equals bit for bit the aggregate that chunk's own
// workgroup publishes.  w = conv w0..w3 and bias of the channel, L = log sigma(Lambda).
template <typename IO, typename Acc>
__device__ void scan_chunk_summary(const ScanFwdArgs& p, int b, int ch, int chunk, const float* w,
                                   float L, Acc& Ag, Acc& Hg) {
  const int T = p.T, D = p.D;
  const IO* x = static_cast<const IO*>(p.x);
  const IO* cs = static_cast<const IO*>(p.conv_state);
  const bool conv = p.conv_w != nullptr;
  auto xat = [&](int t) -> float {
    if (t >= 0 && t < T) return Io<IO>::load1(x + (size_t(b) * T + t) * D + ch);
    if (t < 0 && cs) return Io<IO>::load1(cs + (size_t(b) * 3 + 3 + t) * D + ch);
    return 0.f;
  };
  Ag = Acc(1);
  Hg = Acc(0);
  for (int q = 0; q < kTG; ++q) {
    Acc A = Acc(1), H = Acc(0);
    for (int s = 0; s < kFSteps; ++s) {
      const int t = chunk * kFChunk + q * kFSteps + s;
      const bool valid = t < T;
      const float x0 = xat(t);
      float u = x0;
      if (conv) u = conv_u<IO>(w[4], w[0], w[1], w[2], w[3], x0, xat(t - 1), xat(t - 2), xat(t - 3));
      const size_t o = (size_t(b) * T + (valid ? t : 0)) * D + ch;
      const float ga = valid ? p.a[o] : 1.f, gb = valid ? p.beta[o] : 0.f;
      const bool fz = from_z_mode<Acc>(p);
      const float zba = fz ? p.zb_a[ch] : 0.f, zbx = fz ? p.zb_x[ch] : 0.f;
      Acc av, bu;
      scan_elem<Acc>(valid, ga, gb, u, L, p.from_ri, fz, zba, zbx, p.c, av, bu);
      H = fmaA(av, H, bu);
      A = A * av;
    }
    Hg = fmaA(A, Hg, H);
    Ag = A * Ag;
  }
}

// Incoming state of forward chunk k of one channel, with a canonical result: walk back over
// chunks k-1, k-2, ... to the nearest published inclusive state (or to the chain's initial
// state h0), then apply the aggregates of the chunks in between forward in time order,
// h <- fma(A_j, h, H_j).  Every inclusive state is published as that same composition, so
// the carry is bitwise the one a strictly sequential chain computes, whatever the timing.
// A chunk whose aggregate has not appeared after `direct_polls` polls has its summary
// computed here from memory instead (the same bits its own workgroup would publish): the
// walk never depends on a workgroup that has not started, so the kernel cannot deadlock
// whatever order the hardware runs workgroups in.  direct_polls < 0 ignores everything
// published and computes every summary directly (a test of that path).
template <typename IO, typename Acc>
__device__ Acc scan_lookback(const ScanFwdArgs& p, const typename Words<Acc>::W* incl,
                             const typename Words<Acc>::W* aggA, const typename Words<Acc>::W* aggH,
                             size_t BD, int b, int ch, int k, const float* w, float L, Acc* bufA,
                             Acc* bufH) {
  typedef Words<Acc> Wd;
  const bool use_published = p.direct_polls >= 0;
  int j = k - 1, n = 0, polls = 0;
  bool have = false;
  Acc h = Acc(0);
  while (j >= 0 && use_published) {
    const typename Wd::W vi = peek<Acc>(incl + size_t(j) * BD);
    if (vi != Wd::kEmpty) {
      h = Wd::val(vi);
      have = true;
      break;
    }
    const typename Wd::W va = peek<Acc>(aggA + size_t(j) * BD);
    const typename Wd::W vh = peek<Acc>(aggH + size_t(j) * BD);
    const bool got = va != Wd::kEmpty && vh != Wd::kEmpty;
    if (got || ++polls > p.direct_polls) {
      if (n < kWindow) {
        if (got) {
          bufA[n] = Wd::val(va);
          bufH[n] = Wd::val(vh);
        } else {
          scan_chunk_summary<IO, Acc>(p, b, ch, j, w, L, bufA[n], bufH[n]);
        }
      }
      ++n;
      --j;
      polls = 0;
      continue;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!use_published) n = k;      // walk straight to the initial state
  if (!have) h = p.h0 ? Acc(p.h0[size_t(b) * p.D + ch]) : Acc(0);
  // positions k-n .. k-1 in time order; position k-1-i is the i-th collected
  for (int i = n - 1; i >= 0; --i) {
    Acc A, H;
    if (i < kWindow && use_published) {
      A = bufA[i];
      H = bufH[i];
    } else {
      const int pos = k - 1 - i;
      const typename Wd::W va = use_published ? peek<Acc>(aggA + size_t(pos) * BD) : Wd::kEmpty;
      const typename Wd::W vh = use_published ? peek<Acc>(aggH + size_t(pos) * BD) : Wd::kEmpty;
      if (va != Wd::kEmpty && vh != Wd::kEmpty) {
        A = Wd::val(va);
        H = Wd::val(vh);
      } else {
        scan_chunk_summary<IO, Acc>(p, b, ch, pos, w, L, A, H);
      }
    }
    h = fmaA(A, h, H);
  }
  return h;
}

template <typename IO, typename Acc>
__global__ __launch_bounds__(256, sizeof(Acc) == 4 ? 4 : 2) void scan_fwd_kernel(ScanFwdArgs p) {
  typedef typename Words<Acc>::W W;
  __shared__ Acc sA[kTG][kCh], sH[kTG][kCh];
  __shared__ Acc sCarry[kCh];
  __shared__ Acc sLb[kCh][2][kWindow];
  __shared__ float4 sW[5][kCh / 4];          // conv w0..w3 and bias of the tile's channels
  __shared__ float4 sL[kCh / 4];             // log sigma(Lambda) (gates from r, i or z)
  __shared__ float4 sZ[2][kCh / 4];          // the biases of the from_z mode

  const int B = p.B, T = p.T, D = p.D;
  const int tid = threadIdx.x;
  // Tile of this workgroup: group grp = blockIdx mod G owns the chains grp, grp + G, ...
  // and its workgroups take their tiles time level by time level, so the tile a workgroup
  // waits on always has a lower index (and the look-back never depends on a workgroup that
  // has not started: see scan_lookback).
  const int G = p.groups, grp = blockIdx.x % G;
  const int NB = D / kCh;
  const int per_level = B * NB / G;
  const int tk = int(blockIdx.x) / G;
  const int chunk = tk / per_level;
  const int chain = grp + G * (tk % per_level);
  const int b = chain / NB, d0 = (chain % NB) * kCh;
  const int nchunks = scan_fwd_chunks(T);
  const int t0 = chunk * kFChunk;
  const int cg = tid & 15, tg = tid >> 4;
  const int d = d0 + 4 * cg;
  const int tf = t0 + tg * kFSteps;         // this thread's first step
  const size_t BD = size_t(B) * D;
  const bool conv = p.conv_w != nullptr;

  // ---- every load of the tile first: gates of the 4 steps, then x rows tf-3 .. tf+3.
  // Addresses are a tile base (uniform, in scalar registers) plus a 32-bit byte offset per
  // lane, so a load needs one offset register instead of a 64-bit address.
  const size_t tbase = (size_t(b) * T + t0) * D + d0;      // element (b, t0, d0)
  const char* ta = reinterpret_cast<const char*>(p.a + tbase);
  const char* tbeta = reinterpret_cast<const char*>(p.beta + tbase);
  const uint32_t lane_g = (uint32_t(tg * kFSteps) * uint32_t(D) + uint32_t(4 * cg)) * 4u;
  float4 ga[kFSteps], gb[kFSteps];
#pragma unroll
  for (int s = 0; s < kFSteps; ++s) {
    if (tf + s < T) {
      const uint32_t o = lane_g + uint32_t(s) * uint32_t(D) * 4u;
      ga[s] = load_once4(ta + o);
      gb[s] = load_once4(tbeta + o);
    }
  }
  // x rows from a base at row max(t0 - 3, 0) of the sequence, so every row t >= 0 the tile
  // reads sits at a non-negative offset; rows t < 0 come from the conv history
  const int xrow0 = t0 >= 3 ? t0 - 3 : 0;
  const char* tx = reinterpret_cast<const char*>(static_cast<const IO*>(p.x) +
                                                 ((size_t(b) * T + xrow0) * D + d0));
  const IO* cs = static_cast<const IO*>(p.conv_state);
  Raw4<IO> xr[kFSteps + 3];                  // xr[k] holds x at step tf - 3 + k
#pragma unroll
  for (int k = 0; k < kFSteps + 3; ++k) {
    const int t = tf - 3 + k;
    xr[k].zero();
    if (k < 3 && !conv) continue;            // without the conv only x_t itself is used
    if (t >= 0 && t < T) {
      const uint32_t o = (uint32_t(t - xrow0) * uint32_t(D) + uint32_t(4 * cg)) * uint32_t(sizeof(IO));
      xr[k].load(reinterpret_cast<const IO*>(tx + o));
    } else if (t < 0 && cs) {
      xr[k].load(cs + (size_t(b) * 3 + 3 + t) * D + d);
    }
  }
  // per-channel constants through LDS (one lane per channel), which keeps them out of the
  // registers of every thread
  if (tid < kCh) {
    const int c = d0 + tid;
    float wk[4] = {0.f, 0.f, 0.f, 0.f}, bias = 0.f, L = 0.f;
    if (conv) {
      const IO* w = static_cast<const IO*>(p.conv_w);
#pragma unroll
      for (int q = 0; q < 4; ++q) wk[q] = Io<IO>::load1(w + size_t(q) * D + c);
      if (p.conv_b) bias = p.conv_b[c];
    }
    const bool fz = from_z_mode<Acc>(p);
    if (p.from_ri || fz) L = log_sigmoidf(p.lam[c]);
    float* w0f = reinterpret_cast<float*>(&sW[0][0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) w0f[q * kCh + tid] = wk[q];
    w0f[4 * kCh + tid] = bias;
    reinterpret_cast<float*>(sL)[tid] = L;
    if (sizeof(Acc) == 8) {
      reinterpret_cast<float*>(&sZ[0][0])[tid] = fz ? p.zb_a[c] : 0.f;
      reinterpret_cast<float*>(&sZ[1][0])[tid] = fz ? p.zb_x[c] : 0.f;
    }
  }
  __syncthreads();
  const float4 w0 = sW[0][cg], w1 = sW[1][cg], w2 = sW[2][cg], w3 = sW[3][cg], cb = sW[4][cg];
  const float4 Lv = sL[cg];
  const bool fz = from_z_mode<Acc>(p);
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 zbav = sizeof(Acc) == 8 ? sZ[0][cg] : zero4, zbxv = sizeof(Acc) == 8 ? sZ[1][cg] : zero4;

  // ---- a_t and beta_t u_t of each step (identity map on steps past the end)
  Acc av[kFSteps][4], bu[kFSteps][4];
#pragma unroll
  for (int s = 0; s < kFSteps; ++s) {
    const bool valid = tf + s < T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float u = xr[s + 3].get(j);
      if (conv)
        u = conv_u<IO>(f4get(cb, j), f4get(w0, j), f4get(w1, j), f4get(w2, j), f4get(w3, j),
                       xr[s + 3].get(j), xr[s + 2].get(j), xr[s + 1].get(j), xr[s].get(j));
      scan_elem<Acc>(valid, f4get(ga[s], j), f4get(gb[s], j), u, f4get(Lv, j), p.from_ri, fz,
                     f4get(zbav, j), f4get(zbxv, j), p.c, av[s][j], bu[s][j]);
    }
  }

  // ---- local summary of this thread's steps: h -> A h + H
  Acc A[4], H[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { A[j] = Acc(1); H[j] = Acc(0); }
#pragma unroll
  for (int s = 0; s < kFSteps; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      H[j] = fmaA(av[s][j], H[j], bu[s][j]);
      A[j] = A[j] * av[s][j];
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) { sA[tg][4 * cg + j] = A[j]; sH[tg][4 * cg + j] = H[j]; }
  __syncthreads();

  if (tid < kCh) {
    // One lane per channel (the first wave): tile aggregate, publish, look back, publish
    // the inclusive state.  The 64 look-backs run side by side, so the tile pays for one
    // chain of polls instead of four in a row.
    const int c = 4 * (tid & 15) + (tid >> 4);
    Acc Ag = Acc(1), Hg = Acc(0);
#pragma unroll
    for (int q = 0; q < kTG; ++q) {
      Hg = fmaA(sA[q][c], Hg, sH[q][c]);
      Ag = sA[q][c] * Ag;
    }
    W* incl = static_cast<W*>(p.status);
    W* aggA = incl + size_t(nchunks) * BD;
    W* aggH = aggA + size_t(nchunks) * BD;
    const size_t base = size_t(b) * D + d0 + c;
    Acc carry;
    if (chunk > 0) {
      publish<Acc>(aggA + size_t(chunk) * BD + base, Ag);
      publish<Acc>(aggH + size_t(chunk) * BD + base, Hg);
      const float* wf = reinterpret_cast<const float*>(&sW[0][0]);
      const float wc[5] = {wf[c], wf[kCh + c], wf[2 * kCh + c], wf[3 * kCh + c], wf[4 * kCh + c]};
      carry = scan_lookback<IO, Acc>(p, incl + base, aggA + base, aggH + base, BD, b, d0 + c,
                                     chunk, wc, reinterpret_cast<const float*>(sL)[c], sLb[c][0],
                                     sLb[c][1]);
    } else {
      carry = p.h0 ? Acc(p.h0[base]) : Acc(0);
    }
    publish<Acc>(incl + size_t(chunk) * BD + base, fmaA(Ag, carry, Hg));
    sCarry[c] = carry;
  }
  // exclusive prefix of the time groups before this one
  Acc Ap[4], Hp[4];
  compose_groups<Acc>(sA, sH, 4 * cg, 0, tg, 1, Ap, Hp);
  __syncthreads();

  // ---- re-run the 4 steps from the exact incoming state; write y (and every h_t)
  Acc h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = fmaA(Ap[j], sCarry[4 * cg + j], Hp[j]);
  IO* y = static_cast<IO*>(p.y);
  Acc* h_all = static_cast<Acc*>(p.h_all);
#pragma unroll
  for (int s = 0; s < kFSteps; ++s) {
    const int t = tf + s;
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = fmaA(av[s][j], h[j], bu[s][j]);
    if (t < T) {
      const size_t o = (size_t(b) * T + t) * D + d;
      const float4 hf = make_float4(float(h[0]), float(h[1]), float(h[2]), float(h[3]));
      if (y) Io<IO>::store4_once(y + o, hf);
      if (h_all) {   // read once, by the reverse scan: non-temporal like y
#pragma unroll
        for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(h[j], h_all + o + j);
      }
      if (t == T - 1 && p.h_T) *reinterpret_cast<float4*>(p.h_T + size_t(b) * D + d) = hf;
    }
  }

}

template <typename IO, typename Acc>
hipError_t launch_scan_fwd(const ScanFwdArgs& a_in, hipStream_t s) {
  ScanFwdArgs a = a_in;
  if (a.from_z && sizeof(Acc) != 8) return hipErrorInvalidValue;   // fp32 I/O only
  if (!a.prefilled) {
    const size_t words = 3ull * scan_fwd_chunks(a.T) * size_t(a.B) * a.D * sizeof(Acc) / 4;
    const hipError_t e =
        launch_fill_status(static_cast<uint32_t*>(a.status), words, a.counter, kCounterWords, s);
    if (e != hipSuccess) return e;
  }
  const int chains = a.B * (a.D / kCh);
  a.groups = scan_groups(chains);
  const int tiles = scan_fwd_chunks(a.T) * chains;
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
  // log sigma(Lambda) of the 4 channels in the state's precision (a_t and m_t below too)
  Acc Lv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) Lv[j] = log_sigmoid_acc<Acc>(p.lam[d + j]);
  auto row_of = [&](int s) { return size_t(b) * T + (t0 + tg * kSteps + s); };
  auto valid = [&](int s) { return t0 + tg * kSteps + s < T; };
  // a_t of 4 channels from r_t (identity a = 1 on padded steps)
  auto gate_a = [&](const float4& r, bool ok, int j) -> Acc {
    return ok ? Acc(gate_am(f4get(r, j), Lv[j], p.c).a) : Acc(1);
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
                                       sLb[cg][0], sLb[cg][1], p.max_polls, p.stall);
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
  const Acc cL[4] = {Acc(p.c) * Lv[0], Acc(p.c) * Lv[1], Acc(p.c) * Lv[2], Acc(p.c) * Lv[3]};
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
      const auto gt = gate_am(f4get(cur.r, j), Lv[j], p.c);
      const Acc a = ok ? Acc(gt.a) : Acc(1), m = ok ? Acc(gt.m) : Acc(0);
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
                                          scan_status_bytes(a.B, a.T, a.D, sizeof(Acc)) / 4,
                                          a.counter, kCounterWords, s);
  if (e != hipSuccess) return e;
  const int tiles = scan_chunks(a.T) * a.B * (a.D / kCh);
  scan_bwd_kernel<IO, Acc><<<tiles, 256, 0, s>>>(a);
  return hipGetLastError();
}
template hipError_t launch_scan_bwd<float, double>(const ScanBwdArgs&, hipStream_t);
template hipError_t launch_scan_bwd<bf16_t, float>(const ScanBwdArgs&, hipStream_t);

}  // namespace rglru
