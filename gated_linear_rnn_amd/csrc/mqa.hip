// Local (sliding-window) multi-query attention (Griffin model-architecture page, sections
// "Global multi-query attention" and "Local sliding-window attention"): H query heads of
// width 128 share one key head and one value head; query t attends to the keys at the W
// most recent positions up to and including its own, with weights softmax(q.k / sqrt(128)).
//
// bf16 kernel.  A workgroup owns 64 consecutive query positions of one sequence and 4
// heads (256 queries that all read the same keys: the multi-query sharing), and walks the
// keys of their windows in tiles of 64.  Each of the 8 waves owns 32 queries (one head,
// 32 positions).  Per key tile:
//   S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16, K from LDS as the A operand,
//   the wave's Q fragments held in registers as the B operand for the whole walk), so each
//   lane ends up holding the scores of ONE query (its column) against 32 keys and the
//   partner lane l^32 the other 32: the online softmax (running max m, running sum l) is
//   lane-local apart from one max exchange with the partner per tile;
//   O^T += V^T P^T on the matrix cores, P^T taken straight from the score registers as the
//   B operand.  The B-operand k order of a lane's scores is a fixed permutation of the keys
//   (bits 2 and 3 of the key index within each group of 16 swapped), so V^T is written
//   into LDS in that same permuted order.
// O^T's accumulator also has one query per lane, so the final 1/l scaling is lane-local.
// K tiles arrive by global_load_lds DMA (16-byte chunks XOR-swizzled by row), V tiles
// through registers, transposed into LDS; both double-buffered so the next tile loads
// while the current one is processed.
#include "gemm_core.h"
#include "kernels.h"

namespace rglru {

constexpr int kDh = 128;                   // head width
constexpr int kHB = 4;                     // heads per workgroup
constexpr int kMqaWaves = 8;               // waves per workgroup (4 measured ~5% slower)
constexpr int kKeys = 64;                  // keys per tile
constexpr int kKBytes = kKeys * kDh * 2;   // K tile: 64 rows x 256 B
constexpr int kVBytes = kDh * kKeys * 2;   // V^T tile: 128 rows x 128 B
constexpr int kBuf = kKBytes + kVBytes;

template <int V> struct BufTag { static constexpr int value = V; };

// position of key j (0..63) in a V^T row: bits 2 and 3 swapped (an involution)
__device__ __forceinline__ int vt_pos(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}
// byte offset of (dim d, position pos) in a V^T tile: 8 chunks of 16 B per 128-B row,
// chunk c of row d stored at c ^ (((d >> 1) ^ (d >> 4)) & 7)
__device__ __forceinline__ int vt_off(int d, int pos) {
  return d * 128 + (((pos >> 3) ^ ((d >> 1) ^ (d >> 4))) & 7) * 16 + (pos & 7) * 2;
}

// NW waves: NW / 4 blocks of 32 positions x 4 heads.
template <int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void mqa_fwd_bf16_kernel(MqaArgs p) {
  constexpr int kQPos = 32 * (NW / 4);       // query positions per workgroup
  // Two tile buffers: tile kt is read from one while tile kt + 1 is written into the other.
  // The loop below is unrolled by two so that each copy of the tile step names its buffers
  // at compile time (the LDS addresses become constant offsets).
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[kBuf];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H, T = p.T, S = p.S;
  const int HG = (H + kHB - 1) / kHB;
  const int TB = (T + kQPos - 1) / kQPos;
  int bid = blockIdx.x;
  const int hg = bid % HG;
  bid /= HG;
  const int tb = bid % TB;
  const int b = bid / TB;
  const int t0 = tb * kQPos;
  const int half = lane >> 5, col = lane & 31;

  // this lane's query: head hg*4 + (wave & 3), position t0 + 32 (wave >> 2) + col
  const int head = hg * kHB + (wave & 3);
  const int t = t0 + 32 * (wave >> 2) + col;
  const bool qok = head < H && t < T;
  const int hq = min(head, H - 1), tq = min(t, T - 1);
  const long qpos = long(p.q_pos0) + t;       // absolute position of the query

  // key range of the workgroup: kv positions in (first query - W, last query]
  const int tlast = min(t0 + kQPos, T) - 1;
  const long lo_pos = long(p.q_pos0) + t0 - p.window + 1;
  const int s_lo = int(max(0L, lo_pos - p.kv_pos0));
  const int s_hi = int(min(long(S) - 1, long(p.q_pos0) + tlast - p.kv_pos0));
  const int ntiles = s_hi >= s_lo ? (s_hi - s_lo + kKeys) / kKeys : 0;

  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + size_t(b) * S * kDh;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + size_t(b) * S * kDh;

  // Q fragments (B operand of S^T = K Q^T): dims 16 ks + 8 half .. +8 of this lane's query
  bf16x8_t qf[8];
  {
    const bf16_t* qrow = static_cast<const bf16_t*>(p.q) + (size_t(b) * T + tq) * size_t(H) * kDh +
                         size_t(hq) * kDh + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * ks);
  }

  // ---- tile loads
  auto load_k = [&](int kt, unsigned char* dst) {   // DMA: 16 wave instructions of 1 KB each
#pragma unroll
    for (int i = 0; i < 16 / NW; ++i) {
      const int blk = i * NW + wave;
      const int row = blk * 4 + (lane >> 4), pc = lane & 15;
      const int s = min(s_lo + kt * kKeys + row, s_hi);
      const bf16_t* src = kg + size_t(s) * kDh + ((pc ^ (row & 15)) * 8);
      __builtin_amdgcn_global_load_lds((void*)src, (void*)(dst + blk * 1024), 16, 0, 0);
    }
  };
  // V: thread -> key pairs (2 kp, 2 kp + 1) (adjacent positions of V^T), dims 8 dc .. +8;
  // 512 pair-chunks per tile, 512 / (64 NW) per thread
  constexpr int VIT = 8 / NW;
  uint4 vreg[VIT][2];
  const int vdc = tid & 15;
  auto fetch_v = [&](int kt) {
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int vkp = it * (NW * 4) + (tid >> 4);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int s = min(s_lo + kt * kKeys + 2 * vkp + i, s_hi);
        vreg[it][i] = *reinterpret_cast<const uint4*>(vg + size_t(s) * kDh + vdc * 8);
      }
    }
  };
  auto store_v = [&](unsigned char* buf) {   // transpose into V^T, keys in the permuted order
    unsigned char* vt = buf + kKBytes;
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int vkp = it * (NW * 4) + (tid >> 4);
      const int pos = vt_pos(2 * vkp);   // even; key 2 kp + 1 sits at pos + 1
      const uint32_t a[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
      const uint32_t c[4] = {vreg[it][1].x, vreg[it][1].y, vreg[it][1].z, vreg[it][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (a[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (c[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(vt + vt_off(vdc * 8 + e, pos)) = lo | (hi << 16);
      }
    }
  };

  f32x16_t acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.f;
  float m_run = -1e30f, l_run = 0.f;          // running max (log2 domain) and partial sum

  if (ntiles > 0) {
    load_k(0, lds0);
    fetch_v(0);
    store_v(lds0);
  }
  __syncthreads();
  // one key tile: compute from buffer CUR while the next tile is loaded into the other one
  // (the buffer is a compile-time choice, so each of the two copies addresses one array)
  auto tile = [&](int kt, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    const unsigned char* cur = CUR == 0 ? lds0 : lds1;
    unsigned char* nxt = CUR == 0 ? lds1 : lds0;
    const bool more = kt + 1 < ntiles;
    // Nothing is in flight here after the first tile (each tile ends waiting for its DMA),
    // but on the first one the Q fragment loads may be: settle them before the next tile's
    // loads are issued, so that the compiler's wait before the first K fragment read does
    // not also cover those loads.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (more) {
      load_k(kt + 1, nxt);
      fetch_v(kt + 1);
    }
    const unsigned char* ks_lds = cur;
    const unsigned char* vt_lds = cur + kKBytes;

    // ---- S^T = K Q^T: two 32-key blocks
    f32x16_t acc_s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_s[kb][v] = 0.f;
      const int row = kb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int c = 2 * ks + half;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ks_lds + row * 256 + ((c ^ (row & 15)) * 16));
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc_s[kb], 0, 0, 0);
      }
    }

    // ---- mask, online softmax (log2 domain).  Key j of the tile is allowed when
    // j_lo < j <= j_hi (in the window, not in the future, inside the key range); a tile
    // that every query of the workgroup sees whole skips the mask.
    const int sbase = s_lo + kt * kKeys;
    const long kfirst = long(p.kv_pos0) + sbase, klast = kfirst + kKeys - 1;
    const bool whole = sbase + kKeys - 1 <= s_hi && klast <= long(p.q_pos0) + t0 &&
                       kfirst > long(p.q_pos0) + t0 + kQPos - 1 - p.window;
    // (raw scores: the 1/sqrt(128) log2(e) scale is folded into the exponent below)
    float mx = -INFINITY;
    if (whole) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, acc_s[kb][v]);
    } else {
      const int rel = int(qpos - p.kv_pos0 - sbase);       // the query's own key index
      const int j_hi = min(rel, s_hi - sbase) - 4 * half;
      const int j_lo = rel - p.window - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = kb * 32 + 8 * (v >> 2) + (v & 3);  // key index minus 4 half
          const bool ok = j <= j_hi && j > j_lo;
          const float sc = ok ? acc_s[kb][v] : -INFINITY;
          acc_s[kb][v] = sc;
          mx = fmaxf(mx, sc);
        }
    }
    {
      const WaveHalves mh = wave_halves(mx);       // this lane's and the partner lane's max
      mx = fmaxf(mh.lo, mh.hi);
    }
    mx = fmaxf(mx * p.scale_log2, -1e30f);                 // log2 domain; -1e30: nothing valid
    // The reference max m_run only moves when the tile max exceeds it by more than 8 (in
    // log2 units): the weights exp2(s - m_run) then stay below 2^8, exact enough in fp32,
    // and the rescaling of O and l, which needs a new m_run, is mostly skipped.  The final
    // division by l uses the same reference, so the result does not depend on it.
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
        const float e = __builtin_amdgcn_exp2f(fmaf(acc_s[kb][v], p.scale_log2, -m_run));
        lsum += e;
        pf[kb * 2 + (v >> 3)][v & 7] = (__bf16)e;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T: four 32-dim blocks, four 16-key steps
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vt_lds + vt_off(d, 16 * j + 8 * half));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], acc_o[db], 0, 0, 0);
      }
    }
    if (more) store_v(nxt);
    __syncthreads();   // the next tile is in LDS; every wave is done with this one
  };
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile(kt, BufTag<0>{});
    if (kt + 1 < ntiles) tile(kt + 1, BufTag<1>{});
  }

  // ---- normalise and store: lane = query, dims 32 db + 8 g + 4 half + 0..3
  const WaveHalves lh = wave_halves(l_run);
  const float l_tot = lh.lo + lh.hi;   // this lane's and the partner lane's sum
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qok) {
    bf16_t* orow = static_cast<bf16_t*>(p.o) + (size_t(b) * T + t) * size_t(H) * kDh + size_t(head) * kDh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * half;
        uint2 w;
        w.x = uint32_t(f2bf(acc_o[db][4 * g + 0] * inv)) | (uint32_t(f2bf(acc_o[db][4 * g + 1] * inv)) << 16);
        w.y = uint32_t(f2bf(acc_o[db][4 * g + 2] * inv)) | (uint32_t(f2bf(acc_o[db][4 * g + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
  }
}

// fp32 I/O: one thread per (sequence, position, head), two passes over the window's keys in
// fp64 (max, then weights and the weighted sum of v).  Latency-bound; serves the
// reference-precision path at small sizes.
__global__ __launch_bounds__(128) void mqa_fwd_f32_kernel(MqaArgs p) {
  const int H = p.H, T = p.T, S = p.S;
  const size_t n = size_t(p.B) * T * H;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int head = int(idx % H);
  const int t = int((idx / H) % T);
  const int b = int(idx / (size_t(H) * T));
  const float* q = static_cast<const float*>(p.q) + idx * kDh;
  const float* kb = static_cast<const float*>(p.k) + size_t(b) * S * kDh;
  const float* vb = static_cast<const float*>(p.v) + size_t(b) * S * kDh;
  const long qpos = long(p.q_pos0) + t;
  const int s_lo = int(max(0L, qpos - p.window + 1 - p.kv_pos0));
  const int s_hi = int(min(long(S) - 1, qpos - p.kv_pos0));
  const double scale = 1.0 / sqrt(double(kDh));
  double mx = -1e300;
  for (int s = s_lo; s <= s_hi; ++s) {
    double dot = 0.0;
    for (int d = 0; d < kDh; ++d) dot = fma(double(q[d]), double(kb[size_t(s) * kDh + d]), dot);
    mx = fmax(mx, dot * scale);
  }
  double acc[kDh];
  for (int d = 0; d < kDh; ++d) acc[d] = 0.0;
  double l = 0.0;
  for (int s = s_lo; s <= s_hi; ++s) {
    double dot = 0.0;
    for (int d = 0; d < kDh; ++d) dot = fma(double(q[d]), double(kb[size_t(s) * kDh + d]), dot);
    const double w = exp(dot * scale - mx);
    l += w;
    for (int d = 0; d < kDh; ++d) acc[d] = fma(w, double(vb[size_t(s) * kDh + d]), acc[d]);
  }
  float* o = static_cast<float*>(p.o) + idx * kDh;
  for (int d = 0; d < kDh; ++d) o[d] = l > 0.0 ? float(acc[d] / l) : 0.f;
}

hipError_t launch_mqa_fwd(const MqaArgs& a, bool bf16, hipStream_t s) {
  if (bf16) {
    constexpr int NW = kMqaWaves;
    const int HG = (a.H + kHB - 1) / kHB, TB = (a.T + 32 * (NW / 4) - 1) / (32 * (NW / 4));
    mqa_fwd_bf16_kernel<NW><<<a.B * TB * HG, NW * 64, 0, s>>>(a);
  } else {
    const size_t n = size_t(a.B) * a.T * a.H;
    mqa_fwd_f32_kernel<<<int((n + 127) / 128), 128, 0, s>>>(a);
  }
  return hipGetLastError();
}

// RoPE for fp32 I/O (the bf16 path rotates in the projection GEMM's epilogue): pair
// (2i, 2i+1) of every 128-wide head vector of row m (position pos0 + m % T) rotated by the
// angle pos * 10000^(-2i/128), evaluated in fp64.  x [M, ncols], ncols % 128 == 0.
__global__ __launch_bounds__(256) void rope_f32_kernel(float* x, int M, int ncols, int T, int pos0) {
  const size_t pairs = size_t(M) * (ncols / 2);
  for (size_t o = size_t(blockIdx.x) * blockDim.x + threadIdx.x; o < pairs;
       o += size_t(gridDim.x) * blockDim.x) {
    const int m = int(o / (ncols / 2));
    const int c2 = int(o % (ncols / 2));
    const int i = c2 % (kDh / 2);
    const double ang = double(pos0 + m % T) * pow(10000.0, -2.0 * i / kDh);
    double sn, cs;
    sincos(ang, &sn, &cs);
    float* e = x + size_t(m) * ncols + 2 * c2;
    const double ev = e[0], od = e[1];
    e[0] = float(ev * cs - od * sn);
    e[1] = float(ev * sn + od * cs);
  }
}

hipError_t launch_rope_f32(float* x, int M, int ncols, int T, int pos0, hipStream_t s) {
  const size_t pairs = size_t(M) * (ncols / 2);
  size_t blocks = (pairs + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  rope_f32_kernel<<<int(blocks), 256, 0, s>>>(x, M, ncols, T, pos0);
  return hipGetLastError();
}

}  // namespace rglru
