// C ABI of librglru.so: argument validation, workspace carving and launch orchestration
// on the caller's stream.  Every entry point validates all arguments before the first
// HIP call and never allocates device memory.  Declarations and the contract of each
// entry point are in include/rglru.h.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "../../include/rglru.h"
#include "kernels.h"
#include "rglru_device.h"
#include "rglru_testing.h"

namespace rglru {
const Knobs kDefaultKnobs = {0, kDirectPolls, kMaxPolls, 0};
}

using namespace rglru;

namespace {

constexpr size_t kAlign = 256;

size_t io_bytes(rglru_dtype io) { return io == RGLRU_BF16 ? 2 : 4; }
// Scan state precision: fp32 for bf16 I/O, fp64 for fp32 I/O.
int acc_bytes(rglru_dtype io) { return io == RGLRU_BF16 ? 4 : 8; }
bool io_ok(int io) { return io == RGLRU_F32 || io == RGLRU_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bump allocator over the caller's workspace; with base == nullptr it only measures.
struct Carver {
  unsigned char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<unsigned char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    used = (used + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

int shape_status(int B, int T, int D) {
  if (B <= 0 || T <= 0 || D <= 0) return RGLRU_EINVAL;
  if (D % 64 != 0) return RGLRU_ESHAPE;
  if (int64_t(B) * T * D >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  return RGLRU_OK;
}

bool c_ok(float c) { return c >= 0.f && isfinite(c); }

#define RG_CHECK(expr)                                   \
  do {                                                   \
    if ((expr) != hipSuccess) return RGLRU_EHIP;         \
  } while (0)

// ------------------------------------------------------------------ forward
// bf16 I/O: u, then the fused RG-LRU kernel's look-back status and counters.
// fp32 I/O: u, a, beta (the unfused gates, or the raw projections when the scan forms the
// gates) and the scan's look-back status and counter.
struct FwdWs {
  void* u;
  float* a;      // unfused path: a (fp32 io: z^a, then a in place, or z^a for the scan)
  float* beta;   // unfused path: beta (fp32 io: z^x, then beta in place, or z^x for the scan)
  void* status;
  uint32_t* counter;
  float* tail;   // bf16 unfused path: the gate GEMM's split-tail partials
};

// Which form the RG-LRU layer takes.  fp32 I/O: always the unfused gates + scan.  bf16: the
// fused kernel, except where its tiles (256 steps x 128 channels, lru_tiles of them) leave
// the last of two or more rounds of 256 CUs at most 60% full; the unfused form then fills
// its rounds (the gate GEMM splits the K loop of its own partly filled last round; the scan
// is memory-bound) and is faster.  A pure function of the shape, so the workspace size and
// the bits of every call follow it.
bool lru_unfused(int B, int T, int D, rglru_dtype io) {
  if (io != RGLRU_BF16) return true;
  const long tiles = lru_tiles(B, T, D), rem = tiles % 256;
  return rem != 0 && rem * 5 <= 256 * 3;
}

// The counter words every chained-scan workspace starts with (ticket counters, stall flag).
uint32_t* carve_counters(Carver& cv) { return cv.take<uint32_t>(kCounterWords); }

// The RG-LRU layer's scratch after the counters and u.  `fused`: the caller always runs the
// fused kernel on bf16 (the recurrent block's gated form).
void carve_lru(Carver& cv, FwdWs& w, int B, int T, int D, rglru_dtype io, bool fused = false) {
  const size_t n = size_t(B) * T * D;
  w.a = w.beta = w.tail = nullptr;
  if ((fused && io == RGLRU_BF16) || !lru_unfused(B, T, D, io)) {
    w.status = cv.take<unsigned char>(lru_status_bytes(B, T, D));
  } else {
    w.a = cv.take<float>(n);
    w.beta = cv.take<float>(n);
    w.status = cv.take<unsigned char>(scan_status_bytes(B, T, D, acc_bytes(io)));
    if (io == RGLRU_BF16) {
      const size_t tb = gate_gemm_tail_bytes(B * T, D, D);
      if (tb) w.tail = cv.take<float>(tb / sizeof(float));
    }
  }
}

FwdWs carve_fwd(Carver& cv, int B, int T, int D, rglru_dtype io, bool fused = false) {
  const size_t n = size_t(B) * T * D;
  FwdWs w;
  w.counter = carve_counters(cv);
  w.u = cv.take<unsigned char>(n * io_bytes(io));
  carve_lru(cv, w, B, T, D, io, fused);
  return w;
}

// Look-back status words of the RG-LRU layer's scratch (carve_lru with the same `fused`).
size_t status_fill_words(int B, int T, int D, rglru_dtype io, bool fused = false) {
  const bool unfused = !(fused && io == RGLRU_BF16) && lru_unfused(B, T, D, io);
  return (unfused ? scan_status_bytes(B, T, D, acc_bytes(io)) : lru_status_bytes(B, T, D)) / 4;
}

// The gate projection for M rows: out0/out1 per the epilogue kind.
int gate_projection(rglru_dtype io, GateGemmArgs g, int epi, float* zscratch_a,
                    float* zscratch_x, hipStream_t s) {
  if (io == RGLRU_BF16) {
    RG_CHECK(launch_gate_gemm_bf16(g, epi, s));
    return RGLRU_OK;
  }
  RG_CHECK(launch_gemm_f32_pair(static_cast<const float*>(g.U), static_cast<const float*>(g.Wa),
                                static_cast<const float*>(g.Wx), g.M, g.N, g.K, zscratch_a,
                                zscratch_x, s));
  RG_CHECK(launch_gate_elementwise_f32(g, zscratch_a, zscratch_x, epi, s));
  return RGLRU_OK;
}

// The forward scan over (a, beta): K2.  `prefilled` when the conv launch before it on the
// stream already initialised the look-back status.
// `gz`, when given, makes a and beta the raw projections z^a = u W_a and z^x = u W_x: the
// scan then forms the gates itself (Eq. (2)-(4)) from them, the biases and Lambda.
struct GateZ {
  const float* b_a;
  const float* b_x;
  const float* lam;
  float c;
};
int forward_scan(rglru_dtype io, int B, int T, int D, const void* x, const void* conv_w,
                 const float* conv_b, const void* conv_state_in, const float* a, const float* beta,
                 const float* h0, void* y, float* h_T, void* status, uint32_t* counter,
                 bool prefilled, const Knobs& k, hipStream_t stream, const GateZ* gz = nullptr) {
  ScanFwdArgs sa{};
  sa.B = B; sa.T = T; sa.D = D;
  sa.x = x; sa.conv_w = conv_w; sa.conv_b = conv_b; sa.conv_state = conv_w ? conv_state_in : nullptr;
  sa.a = a; sa.beta = beta; sa.from_ri = false; sa.lam = nullptr; sa.c = 0.f;
  sa.from_z = gz != nullptr;
  if (gz) {
    sa.zb_a = gz->b_a; sa.zb_x = gz->b_x; sa.lam = gz->lam; sa.c = gz->c;
  }
  sa.h0 = h0; sa.y = y; sa.h_all = nullptr; sa.h_T = h_T;
  sa.status = status; sa.counter = counter; sa.prefilled = prefilled;
  sa.direct_polls = k.scan_direct_polls;
  if (io == RGLRU_BF16) RG_CHECK((launch_scan_fwd<bf16_t, float>(sa, stream)));
  else RG_CHECK((launch_scan_fwd<float, double>(sa, stream)));
  return RGLRU_OK;
}

// The RG-LRU layer on the conv output u (Eq. (1)-(4)): the fused kernel, or the gate
// projection then the scan (lru_unfused).  `prefilled`: the launch before it on the stream
// already initialised the look-back status and counters.
int lru_layer(rglru_dtype io, int B, int T, int D, float c, const void* u, const void* W_a,
              const void* W_x, const float* b_a, const float* b_x, const float* lambda,
              const float* h0, void* y, float* h_T, FwdWs& w, bool prefilled, const Knobs& k,
              hipStream_t stream) {
  if ((k.lru_force_fused && io == RGLRU_BF16) || !lru_unfused(B, T, D, io)) {
    LruArgs la{};
    la.u = u; la.Wa = W_a; la.Wx = W_x; la.ba = b_a; la.bx = b_x; la.lam = lambda; la.c = c;
    la.h0 = h0; la.y = y; la.hT = h_T; la.B = B; la.T = T; la.D = D;
    la.status = static_cast<uint32_t*>(w.status); la.counters = w.counter;
    la.ticket_guess = k.lru_ticket_guess; la.max_polls = k.lookback_polls;
    la.stall = w.counter + kStallWord;
    RG_CHECK(launch_lru_fused(la, prefilled, stream));
    return RGLRU_OK;
  }
  if (io == RGLRU_F32 && scan_fwd_tiles(B, T, D) >= 256) {
    // fp32 with a scan that fills the CUs: the two projections in one GEMM launch, the
    // gates formed inside the scan (one launch and one pass over a and beta fewer).  On
    // fewer tiles the scan's per-thread chain is the critical path and the gate math runs
    // faster in the wide elementwise launch below.
    RG_CHECK(launch_gemm_f32_pair(static_cast<const float*>(u), static_cast<const float*>(W_a),
                                  static_cast<const float*>(W_x), B * T, D, D, w.a, w.beta,
                                  stream));
    const GateZ gz{b_a, b_x, lambda, c};
    return forward_scan(io, B, T, D, u, nullptr, nullptr, nullptr, w.a, w.beta, h0, y, h_T,
                        w.status, w.counter, prefilled, k, stream, &gz);
  }
  GateGemmArgs g{};
  g.U = u; g.Wa = W_a; g.Wx = W_x; g.M = B * T; g.N = D; g.K = D;
  g.ba = b_a; g.bx = b_x; g.lam = lambda; g.c = c;
  g.out0 = w.a; g.out1 = w.beta; g.tail_ws = w.tail;
  int st = gate_projection(io, g, kEpiAB, w.a, w.beta, stream);
  if (st != RGLRU_OK) return st;
  return forward_scan(io, B, T, D, u, nullptr, nullptr, nullptr, w.a, w.beta, h0, y, h_T,
                      w.status, w.counter, prefilled, k, stream);
}

struct ScanWs {
  void* status;
  uint32_t* counter;
};
ScanWs carve_scan(Carver& cv, int B, int T, int D, rglru_dtype io) {
  ScanWs w;
  w.counter = carve_counters(cv);
  w.status = cv.take<unsigned char>(scan_status_bytes(B, T, D, acc_bytes(io)));
  return w;
}

// ------------------------------------------------------------------ backward
// What the backward reads of the forward (the chain rule needs u_t, r_t, i_t and h_{t-1}):
// u, the conv output (io), the gates r and i (fp32) and every state h_t (the scan state type).
struct SavedAct {
  void* u;
  float* r;
  float* i;
  void* h_all;
};

SavedAct carve_saved(Carver& cv, int B, int T, int D, rglru_dtype io) {
  const size_t n = size_t(B) * T * D;
  SavedAct a;
  a.u = cv.take<unsigned char>(n * io_bytes(io));
  a.r = cv.take<float>(n);
  a.i = cv.take<float>(n);
  a.h_all = cv.take<unsigned char>(n * acc_bytes(io));
  return a;
}

struct BwdWs {
  SavedAct act;  // recomputed here unless the caller passes the training forward's
  void* dz_hi;   // [M, 2D] (bf16) or fp32 dz
  void* dz_lo;   // [M, 2D] bf16 (bf16 io only)
  void* dzT_hi;  // [2D, Mp]
  void* dzT_lo;
  void* uT;      // [D, Mp]
  void* WT;      // [D, 2D]
  float* du;     // [M, D]
  double* scan_part;
  double* conv_part;
  void* status;
  uint32_t* counter;
  float* tail;   // bf16: split-tail partials of the recompute, input- and weight-gradient products
};

// `recompute`: the backward evaluates the forward itself (rglru_bwd) and holds its
// activations here; without it they come from the caller (rglru_bwd_saved).
BwdWs carve_bwd(Carver& cv, int B, int T, int D, rglru_dtype io, bool recompute = true) {
  const size_t M = size_t(B) * T, n = M * D, Mp = (M + 63) / 64 * 64;
  const size_t eb = io_bytes(io);
  const size_t P = size_t(B) * scan_chunks(T);
  BwdWs w;
  w.counter = carve_counters(cv);
  w.act = recompute ? carve_saved(cv, B, T, D, io) : SavedAct{nullptr, nullptr, nullptr, nullptr};
  w.dz_hi = cv.take<unsigned char>(2 * n * eb);
  w.dz_lo = io == RGLRU_BF16 ? cv.take<unsigned char>(2 * n * eb) : nullptr;
  w.dzT_hi = cv.take<unsigned char>(2 * size_t(D) * Mp * eb);
  w.dzT_lo = io == RGLRU_BF16 ? cv.take<unsigned char>(2 * size_t(D) * Mp * eb) : nullptr;
  w.uT = cv.take<unsigned char>(size_t(D) * Mp * eb);
  w.WT = cv.take<unsigned char>(2 * size_t(D) * D * eb);
  w.du = cv.take<float>(n);
  w.scan_part = cv.take<double>(P * 3 * D);
  w.conv_part = cv.take<double>(P * 5 * D);
  w.status = cv.take<unsigned char>(scan_status_bytes(B, T, D, acc_bytes(io)));
  w.tail = nullptr;
  if (io == RGLRU_BF16) {
    const size_t tb = std::max({plain_gemm_tail_bytes(int(M), D, 2 * D),
                                plain_gemm_tail_bytes(2 * D, D, int(Mp)),
                                recompute ? gate_gemm_tail_bytes(int(M), D, D) : size_t(0)});
    if (tb) w.tail = cv.take<float>(tb / sizeof(float));
  }
  return w;
}

// Scratch of the training forward: the counters, the forward scan's look-back status and the
// gate projection's split-tail partials (bf16).
struct TrainWs {
  uint32_t* counter;
  void* status;
  float* tail;
};

TrainWs carve_train(Carver& cv, int B, int T, int D, rglru_dtype io) {
  TrainWs w;
  w.counter = carve_counters(cv);
  w.status = cv.take<unsigned char>(scan_status_bytes(B, T, D, acc_bytes(io)));
  w.tail = nullptr;
  if (io == RGLRU_BF16) {
    const size_t tb = gate_gemm_tail_bytes(B * T, D, D);
    if (tb) w.tail = cv.take<float>(tb / sizeof(float));
  }
  return w;
}

// The forward as the backward evaluates it, keeping its activations in `a`: u = conv(x) (x
// itself without the conv; the conv launch also initialises the scan's look-back status),
// r and i from the gate projection (kEpiRI epilogue), then the forward scan from (r, i)
// writing every h_t and, where given, y, h_T and the conv state.  *u_out = u.
static int forward_acts(rglru_dtype io, int B, int T, int D, float c, const void* x,
                        const void* conv_w, const float* conv_b, const void* cs, const void* W_a,
                        const void* W_x, const float* b_a, const float* b_x, const float* lambda,
                        const float* h0, const SavedAct& a, float* tail, void* status,
                        uint32_t* counter, void* y, float* h_T, void* conv_state_out,
                        const Knobs& k, hipStream_t stream, const void** u_out) {
  const bool bf = io == RGLRU_BF16;
  const void* u = x;
  bool prefilled = false;
  if (conv_w) {
    uint32_t* fill = static_cast<uint32_t*>(status);
    const size_t words = scan_status_bytes(B, T, D, acc_bytes(io)) / 4;
    if (bf)
      RG_CHECK(launch_conv_fwd<bf16_t>(B, T, D, x, conv_w, conv_b, cs, a.u, conv_state_out, stream,
                                       fill, words, counter));
    else
      RG_CHECK(launch_conv_fwd<float>(B, T, D, x, conv_w, conv_b, cs, a.u, conv_state_out, stream,
                                      fill, words, counter));
    u = a.u;
    prefilled = true;
  }
  GateGemmArgs g{};
  g.U = u; g.Wa = W_a; g.Wx = W_x; g.M = B * T; g.N = D; g.K = D;
  g.ba = b_a; g.bx = b_x; g.lam = lambda; g.c = c;
  g.out0 = a.r; g.out1 = a.i;
  g.tail_ws = tail;
  const int st = gate_projection(io, g, kEpiRI, a.r, a.i, stream);
  if (st != RGLRU_OK) return st;
  ScanFwdArgs sf{};
  sf.B = B; sf.T = T; sf.D = D;
  sf.x = u; sf.conv_w = nullptr; sf.conv_b = nullptr; sf.conv_state = nullptr;   // u is in memory
  sf.a = a.r; sf.beta = a.i; sf.from_ri = true; sf.lam = lambda; sf.c = c;
  sf.h0 = h0; sf.y = y; sf.h_all = a.h_all; sf.h_T = h_T;
  sf.status = status; sf.counter = counter; sf.prefilled = prefilled;
  sf.direct_polls = k.scan_direct_polls;
  if (bf) RG_CHECK((launch_scan_fwd<bf16_t, float>(sf, stream)));
  else RG_CHECK((launch_scan_fwd<float, double>(sf, stream)));
  *u_out = u;
  return RGLRU_OK;
}

// ------------------------------------------------------------------ recurrent block
// bf16 I/O: p, g, u, then the fused RG-LRU layer's scratch; z goes over p (or u).
// fp32 I/O: the [M, 2R] input product, p, g, u, y (later z in place), the layer's scratch.
struct BlockWs {
  float* pq;
  void* p;
  void* g;
  void* y;
  float* tail;   // bf16: the output linear's split-tail partials
  FwdWs lru;
};

BlockWs carve_block(Carver& cv, int B, int T, int D, int R, rglru_dtype io) {
  const size_t n = size_t(B) * T * R;
  BlockWs w;
  w.lru.counter = carve_counters(cv);
  w.pq = io == RGLRU_F32 ? cv.take<float>(2 * n) : nullptr;
  w.tail = io == RGLRU_BF16 ? cv.take<float>(out_gemm_tail_bytes(B * T, D, R) / sizeof(float)) : nullptr;
  w.p = cv.take<unsigned char>(n * io_bytes(io));
  w.g = cv.take<unsigned char>(n * io_bytes(io));
  w.y = io == RGLRU_F32 ? cv.take<unsigned char>(n * io_bytes(io)) : nullptr;
  w.lru.u = cv.take<unsigned char>(n * io_bytes(io));
  carve_lru(cv, w.lru, B, T, R, io, /*fused=*/true);
  return w;
}

int block_shape_status(int B, int T, int D, int R) {
  if (B <= 0 || T <= 0 || D <= 0 || R <= 0) return RGLRU_EINVAL;
  if (D % 64 != 0 || R % 64 != 0) return RGLRU_ESHAPE;
  const int64_t M = int64_t(B) * T;
  if (M * D >= (int64_t(1) << 31) || M * R >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  if (int64_t(2) * R * D >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  return RGLRU_OK;
}

// ------------------------------------------------------------------ gated MLP block
int mlp_shape_status(int B, int T, int D, int MD) {
  if (B <= 0 || T <= 0 || D <= 0 || MD <= 0) return RGLRU_EINVAL;
  if (D % 64 != 0 || MD % 64 != 0) return RGLRU_ESHAPE;
  const int64_t M = int64_t(B) * T;
  if (M * D >= (int64_t(1) << 31) || M * MD >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  if (int64_t(MD) * D >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  return RGLRU_OK;
}

// bf16: h [M, MD] bf16 and the last linear's split-tail partials.  fp32: q1 (then h in
// place) and q2, [M, MD] fp32 each.
struct MlpWs {
  void* h;
  float* q2;
  float* tail;
};
MlpWs carve_mlp(Carver& cv, int B, int T, int D, int MD, rglru_dtype io) {
  const size_t n = size_t(B) * T * MD;
  MlpWs w;
  w.h = cv.take<unsigned char>(n * io_bytes(io));
  w.q2 = io == RGLRU_F32 ? cv.take<float>(n) : nullptr;
  w.tail = io == RGLRU_BF16 ? cv.take<float>(out_gemm_tail_bytes(B * T, D, MD) / sizeof(float)) : nullptr;
  return w;
}

// ------------------------------------------------------------------ local MQA block
constexpr int kHeadDim = 128;

int mqa_shape_status(int B, int T, int D, int window, int pos0) {
  if (B <= 0 || T <= 0 || D <= 0 || window <= 0 || pos0 < 0) return RGLRU_EINVAL;
  if (D % kHeadDim != 0) return RGLRU_ESHAPE;
  const int64_t M = int64_t(B) * T;
  if (M * (D + 2 * kHeadDim) >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  if (int64_t(pos0) + T >= (int64_t(1) << 30)) return RGLRU_ESHAPE;
  return RGLRU_OK;
}

struct MqaWs {
  void* q;
  void* k;
  void* v;
  void* attn;
  float* tail;   // bf16: the output projection's split-tail partials
};
MqaWs carve_mqa(Carver& cv, int B, int T, int D, rglru_dtype io) {
  const size_t M = size_t(B) * T, eb = io_bytes(io);
  MqaWs w;
  w.q = cv.take<unsigned char>(M * D * eb);
  w.k = cv.take<unsigned char>(M * kHeadDim * eb);
  w.v = cv.take<unsigned char>(M * kHeadDim * eb);
  w.attn = cv.take<unsigned char>(M * D * eb);
  w.tail = io == RGLRU_BF16 ? cv.take<float>(out_gemm_tail_bytes(B * T, D, D) / sizeof(float)) : nullptr;
  return w;
}

// ------------------------------------------------------------------ allocation-free decode
// The fixed scratch of rglru_decode_step_noalloc: one array per GPU, held by that GPU until
// the process ends.  Host code never passes `scratch` itself to a kernel (on the host it is
// only a stand-in for the symbol): it uses the device address hipGetSymbolAddress returns,
// looked up once per device with that device current and kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[RGLRU_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// The current device's scratch address (nullptr if the lookup fails).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_dev[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_dev[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    scratch_dev[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

const char* rglru_status_string(int status) {
  switch (status) {
    case RGLRU_OK: return "RGLRU_OK";
    case RGLRU_EINVAL: return "RGLRU_EINVAL: invalid argument (null pointer, non-positive size, misaligned pointer or bad c)";
    case RGLRU_ESHAPE: return "RGLRU_ESHAPE: unsupported shape (D % 64 != 0 or B*T*D >= 2^31)";
    case RGLRU_EDTYPE: return "RGLRU_EDTYPE: unknown I/O dtype";
    case RGLRU_EWORKSPACE: return "RGLRU_EWORKSPACE: workspace missing or too small";
    case RGLRU_EHIP: return "RGLRU_EHIP: HIP launch or runtime error";
    case RGLRU_EINTERNAL: return "RGLRU_EINTERNAL: internal error";
    case RGLRU_ESTALL: return "RGLRU_ESTALL: a chained-scan wait for a predecessor chunk gave up (outputs hold NaN)";
    case RGLRU_ESCRATCH: return "RGLRU_ESCRATCH: the shape needs more than the allocation-free entry point's fixed scratch";
    default: return "unknown rglru status";
  }
}

int conv1d_causal4(int B, int T, int D, rglru_dtype io, const void* x, const void* w,
                   const float* b, const void* state_in, void* u, void* state_out,
                   hipStream_t stream) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !w || !u) return RGLRU_EINVAL;
  for (const void* p : {x, w, (const void*)b, state_in, (const void*)u, (const void*)state_out})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (io == RGLRU_BF16) RG_CHECK(launch_conv_fwd<bf16_t>(B, T, D, x, w, b, state_in, u, state_out, stream));
  else RG_CHECK(launch_conv_fwd<float>(B, T, D, x, w, b, state_in, u, state_out, stream));
  return RGLRU_OK;
}

size_t rglru_fwd_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_fwd(cv, B, T, D, io);
  return cv.used;
}

static int fwd_impl(const Knobs& k, int B, int T, int D, rglru_dtype io, float c, const void* x,
                    const void* conv_w, const float* conv_b, const void* conv_state_in,
                    const void* W_a, const void* W_x, const float* b_a, const float* b_x,
                    const float* lambda, const float* h0, void* y, float* h_T,
                    void* conv_state_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !W_a || !W_x || !b_a || !b_x || !lambda || !y || !c_ok(c)) return RGLRU_EINVAL;
  for (const void* p : {x, conv_w, (const void*)conv_b, conv_state_in, W_a, W_x, (const void*)b_a,
                        (const void*)b_x, (const void*)lambda, (const void*)h0, (const void*)y,
                        (const void*)h_T, (const void*)conv_state_out, (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_fwd_workspace_bytes(B, T, D, io)) return RGLRU_EWORKSPACE;

  // (the fused form's workspace is never larger than the unfused one's, so a forced fused
  // form fits the workspace sized for the shape's own form)
  const bool fused = k.lru_force_fused != 0;
  Carver cv(ws);
  FwdWs w = carve_fwd(cv, B, T, D, io, fused);
  const void* u = x;
  bool prefilled = false;
  if (conv_w) {
    // the conv launch also initialises the layer's look-back status and counters
    uint32_t* fill = static_cast<uint32_t*>(w.status);
    const size_t words = status_fill_words(B, T, D, io, fused);
    if (io == RGLRU_BF16)
      RG_CHECK(launch_conv_fwd<bf16_t>(B, T, D, x, conv_w, conv_b, conv_state_in, w.u, conv_state_out,
                                       stream, fill, words, w.counter));
    else
      RG_CHECK(launch_conv_fwd<float>(B, T, D, x, conv_w, conv_b, conv_state_in, w.u, conv_state_out,
                                      stream, fill, words, w.counter));
    u = w.u;
    prefilled = true;
  }
  return lru_layer(io, B, T, D, c, u, W_a, W_x, b_a, b_x, lambda, h0, y, h_T, w, prefilled, k,
                   stream);
}

int rglru_fwd(int B, int T, int D, rglru_dtype io, float c, const void* x, const void* conv_w,
              const float* conv_b, const void* conv_state_in, const void* W_a, const void* W_x,
              const float* b_a, const float* b_x, const float* lambda, const float* h0, void* y,
              float* h_T, void* conv_state_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(kDefaultKnobs, B, T, D, io, c, x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a,
                  b_x, lambda, h0, y, h_T, conv_state_out, ws, ws_bytes, stream);
}

size_t rglru_lru_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  FwdWs w;
  w.counter = carve_counters(cv);
  carve_lru(cv, w, B, T, D, io);
  return cv.used;
}

int rglru_lru(int B, int T, int D, rglru_dtype io, float c, const void* u, const void* W_a,
              const void* W_x, const float* b_a, const float* b_x, const float* lambda,
              const float* h0, void* y, float* h_T, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!u || !W_a || !W_x || !b_a || !b_x || !lambda || !y || !c_ok(c)) return RGLRU_EINVAL;
  for (const void* p : {u, W_a, W_x, (const void*)b_a, (const void*)b_x, (const void*)lambda,
                        (const void*)h0, (const void*)y, (const void*)h_T, (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_lru_workspace_bytes(B, T, D, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  FwdWs w;
  w.u = nullptr;
  w.counter = carve_counters(cv);
  carve_lru(cv, w, B, T, D, io);
  return lru_layer(io, B, T, D, c, u, W_a, W_x, b_a, b_x, lambda, h0, y, h_T, w, false,
                   kDefaultKnobs, stream);
}

int rglru_gates(int B, int T, int D, rglru_dtype io, float c, const void* u, const void* W_a,
                const void* W_x, const float* b_a, const float* b_x, const float* lambda, float* a,
                float* beta, hipStream_t stream) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!u || !W_a || !W_x || !b_a || !b_x || !lambda || !a || !beta || !c_ok(c)) return RGLRU_EINVAL;
  for (const void* p : {u, W_a, W_x, (const void*)b_a, (const void*)b_x, (const void*)lambda,
                        (const void*)a, (const void*)beta})
    if (!aligned16(p)) return RGLRU_EINVAL;
  GateGemmArgs g{};
  g.U = u; g.Wa = W_a; g.Wx = W_x; g.M = B * T; g.N = D; g.K = D;
  g.ba = b_a; g.bx = b_x; g.lam = lambda; g.c = c;
  g.out0 = a; g.out1 = beta;
  return gate_projection(io, g, kEpiAB, a, beta, stream);
}

size_t rglru_scan_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_scan(cv, B, T, D, io);
  return cv.used;
}

static int scan_impl(const Knobs& k, int B, int T, int D, rglru_dtype io, const void* x,
                     const void* conv_w, const float* conv_b, const void* conv_state_in,
                     const float* a, const float* beta, const float* h0, void* y, float* h_T,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !a || !beta || !y) return RGLRU_EINVAL;
  for (const void* p : {x, conv_w, (const void*)conv_b, conv_state_in, (const void*)a,
                        (const void*)beta, (const void*)h0, (const void*)y, (const void*)h_T,
                        (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_scan_workspace_bytes(B, T, D, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  ScanWs w = carve_scan(cv, B, T, D, io);
  return forward_scan(io, B, T, D, x, conv_w, conv_b, conv_state_in, a, beta, h0, y, h_T,
                      w.status, w.counter, false, k, stream);
}

int rglru_scan(int B, int T, int D, rglru_dtype io, const void* x, const void* conv_w,
               const float* conv_b, const void* conv_state_in, const float* a, const float* beta,
               const float* h0, void* y, float* h_T, void* ws, size_t ws_bytes, hipStream_t stream) {
  return scan_impl(kDefaultKnobs, B, T, D, io, x, conv_w, conv_b, conv_state_in, a, beta, h0, y,
                   h_T, ws, ws_bytes, stream);
}

size_t rglru_decode_workspace_bytes(int B, int D, rglru_dtype io) {
  if (shape_status(B, 1, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  cv.take<unsigned char>(size_t(B) * D * io_bytes(io));
  if (io == RGLRU_F32) {
    cv.take<float>(size_t(B) * D);
    cv.take<float>(size_t(B) * D);
  } else {
    cv.take<unsigned char>(decode_partial_bytes(B, D));
  }
  return cv.used;
}

int rglru_decode_step(int B, int D, rglru_dtype io, float c, const void* x_t, const void* conv_w,
                      const float* conv_b, void* conv_state, const void* W_a, const void* W_x,
                      const float* b_a, const float* b_x, const float* lambda, float* h,
                      void* y_t, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = shape_status(B, 1, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x_t || !W_a || !W_x || !b_a || !b_x || !lambda || !h || !y_t || !c_ok(c)) return RGLRU_EINVAL;
  if (conv_w && !conv_state) return RGLRU_EINVAL;
  for (const void* p : {x_t, conv_w, (const void*)conv_b, (const void*)conv_state, W_a, W_x,
                        (const void*)b_a, (const void*)b_x, (const void*)lambda, (const void*)h,
                        (const void*)y_t, (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_decode_workspace_bytes(B, D, io)) return RGLRU_EWORKSPACE;

  Carver cv(ws);
  void* ubuf = cv.take<unsigned char>(size_t(B) * D * io_bytes(io));
  float* za = io == RGLRU_F32 ? cv.take<float>(size_t(B) * D) : nullptr;
  float* zx = io == RGLRU_F32 ? cv.take<float>(size_t(B) * D) : nullptr;
  float* partial = io == RGLRU_BF16
                       ? reinterpret_cast<float*>(cv.take<unsigned char>(decode_partial_bytes(B, D)))
                       : nullptr;
  const void* u = x_t;
  if (conv_w) {
    if (io == RGLRU_BF16) RG_CHECK(launch_conv_decode<bf16_t>(B, D, x_t, conv_w, conv_b, conv_state, ubuf, stream));
    else RG_CHECK(launch_conv_decode<float>(B, D, x_t, conv_w, conv_b, conv_state, ubuf, stream));
    u = ubuf;
  }
  if (io == RGLRU_BF16) {
    DecodeArgs d{};
    d.u = u; d.Wa = W_a; d.Wx = W_x; d.ba = b_a; d.bx = b_x; d.lam = lambda; d.c = c;
    d.h = h; d.y = y_t; d.partial = partial; d.B = B; d.D = D;
    RG_CHECK(launch_decode_bf16(d, stream));
    return RGLRU_OK;
  }
  GateGemmArgs g{};
  g.U = u; g.Wa = W_a; g.Wx = W_x; g.M = B; g.N = D; g.K = D;
  g.ba = b_a; g.bx = b_x; g.lam = lambda; g.c = c;
  g.u = u; g.h = h; g.y = y_t;
  return gate_projection(io, g, kEpiDecode, za, zx, stream);
}

int rglru_decode_step_noalloc(int B, int D, rglru_dtype io, float c, const void* x_t,
                              const void* conv_w, const float* conv_b, void* conv_state,
                              const void* W_a, const void* W_x, const float* b_a,
                              const float* b_x, const float* lambda, float* h, void* y_t,
                              hipStream_t stream) {
  int st = shape_status(B, 1, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  const size_t need = rglru_decode_workspace_bytes(B, D, io);
  if (need > RGLRU_NOALLOC_SCRATCH_BYTES) return RGLRU_ESCRATCH;
  void* ws = scratch_of_current_device();
  if (!ws) return RGLRU_EHIP;
  return rglru_decode_step(B, D, io, c, x_t, conv_w, conv_b, conv_state, W_a, W_x, b_a, b_x,
                           lambda, h, y_t, ws, RGLRU_NOALLOC_SCRATCH_BYTES, stream);
}

size_t rglru_bwd_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_bwd(cv, B, T, D, io);
  return cv.used;
}

static int bwd_impl(const Knobs& k, int B, int T, int D, rglru_dtype io, float c, const void* x,
                    const void* conv_w, const float* conv_b, const void* conv_state_in,
                    const void* W_a, const void* W_x, const float* b_a, const float* b_x,
                    const float* lambda, const float* h0, const void* dy, const float* dh_T,
                    float* dx, float* dconv_w, float* dconv_b, float* dW_a, float* dW_x,
                    float* db_a, float* db_x, float* dlambda, float* dh0, void* ws,
                    size_t ws_bytes, hipStream_t stream, const void* saved = nullptr,
                    size_t saved_bytes = 0) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !W_a || !W_x || (!saved && (!b_a || !b_x)) || !lambda || !dy || !dx || !dW_a ||
      !dW_x || !db_a || !db_x || !dlambda || !c_ok(c))
    return RGLRU_EINVAL;
  if (conv_w && (!dconv_w || !dconv_b)) return RGLRU_EINVAL;
  for (const void* p : {x, conv_w, (const void*)conv_b, conv_state_in, W_a, W_x, (const void*)b_a,
                        (const void*)b_x, (const void*)lambda, (const void*)h0, dy, (const void*)dh_T,
                        (const void*)dx, (const void*)dconv_w, (const void*)dconv_b,
                        (const void*)dW_a, (const void*)dW_x, (const void*)db_a, (const void*)db_x,
                        (const void*)dlambda, (const void*)dh0, (const void*)ws, saved})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (saved && saved_bytes < rglru_train_saved_bytes(B, T, D, io)) return RGLRU_EINVAL;
  const size_t need = saved ? rglru_bwd_saved_workspace_bytes(B, T, D, io)
                            : rglru_bwd_workspace_bytes(B, T, D, io);
  if (!ws || ws_bytes < need) return RGLRU_EWORKSPACE;

  Carver cv(ws);
  BwdWs w = carve_bwd(cv, B, T, D, io, /*recompute=*/!saved);
  if (saved) {
    Carver sv(const_cast<void*>(saved));
    w.act = carve_saved(sv, B, T, D, io);
  }
  const int M = B * T;
  const int Mp = (M + 63) / 64 * 64;
  const bool bf = io == RGLRU_BF16;
  const void* cs = conv_w ? conv_state_in : nullptr;

  // 1. u, the gates (r, i) and every state h_t: recomputed, or the training forward's
  const void* u = conv_w ? w.act.u : x;
  if (!saved) {
    st = forward_acts(io, B, T, D, c, x, conv_w, conv_b, cs, W_a, W_x, b_a, b_x, lambda, h0, w.act,
                      w.tail, w.status, w.counter, nullptr, nullptr, nullptr, k, stream, &u);
    if (st != RGLRU_OK) return st;
  }

  // 2. reverse scan: dz^a, dz^x, the direct du term, dh0, partial sums
  float* du = conv_w ? w.du : dx;   // without the conv, du is dx
  ScanBwdArgs sb{};
  sb.B = B; sb.T = T; sb.D = D;
  sb.u = u; sb.r = w.act.r; sb.i = w.act.i; sb.h_all = w.act.h_all; sb.h0 = h0;
  sb.dy = dy; sb.dh_T = dh_T; sb.lam = lambda; sb.c = c;
  sb.dz_hi = w.dz_hi; sb.dz_lo = w.dz_lo; sb.du = du; sb.dh0 = dh0;
  sb.partial = w.scan_part; sb.status = w.status; sb.counter = w.counter;
  sb.max_polls = k.lookback_polls; sb.stall = w.counter + kStallWord;
  if (bf) RG_CHECK((launch_scan_bwd<bf16_t, float>(sb, stream)));
  else RG_CHECK((launch_scan_bwd<float, double>(sb, stream)));

  // 3. du += [dz^a dz^x] [W_a; W_x]   (K = 2D; the B operand is [W_a; W_x]^T)
  PlainGemmArgs pg{};
  if (bf) {
    const uint16_t* Wa16 = static_cast<const uint16_t*>(W_a);
    const uint16_t* Wx16 = static_cast<const uint16_t*>(W_x);
    uint16_t* WT = static_cast<uint16_t*>(w.WT);
    RG_CHECK(launch_transpose<uint16_t>(Wa16, D, D, D, WT, 2 * D, D, stream));
    RG_CHECK(launch_transpose<uint16_t>(Wx16, D, D, D, WT + D, 2 * D, D, stream));
  } else {
    float* WT = static_cast<float*>(w.WT);
    RG_CHECK(launch_transpose<float>(static_cast<const float*>(W_a), D, D, D, WT, 2 * D, D, stream));
    RG_CHECK(launch_transpose<float>(static_cast<const float*>(W_x), D, D, D, WT + D, 2 * D, D, stream));
  }
  pg.A = w.dz_hi; pg.A2 = bf ? w.dz_lo : nullptr; pg.Bm = w.WT;
  pg.M = M; pg.N = D; pg.K = 2 * D; pg.lda = 2 * D; pg.ldb = 2 * D; pg.ldc = D;
  pg.C = du; pg.addend = du;
  pg.tail_ws = w.tail;
  if (bf) RG_CHECK(launch_plain_gemm_bf16(pg, stream));
  else RG_CHECK(launch_plain_gemm_f32(pg, stream));

  // 4. dW = dz^T u   (reduction over the B*T rows, zero-padded to Mp)
  if (bf) {
    RG_CHECK(launch_transpose<uint16_t>(static_cast<const uint16_t*>(w.dz_hi), M, 2 * D, 2 * D,
                                        static_cast<uint16_t*>(w.dzT_hi), Mp, Mp, stream));
    RG_CHECK(launch_transpose<uint16_t>(static_cast<const uint16_t*>(w.dz_lo), M, 2 * D, 2 * D,
                                        static_cast<uint16_t*>(w.dzT_lo), Mp, Mp, stream));
    RG_CHECK(launch_transpose<uint16_t>(static_cast<const uint16_t*>(u), M, D, D,
                                        static_cast<uint16_t*>(w.uT), Mp, Mp, stream));
  } else {
    RG_CHECK(launch_transpose<float>(static_cast<const float*>(w.dz_hi), M, 2 * D, 2 * D,
                                     static_cast<float*>(w.dzT_hi), Mp, Mp, stream));
    RG_CHECK(launch_transpose<float>(static_cast<const float*>(u), M, D, D,
                                     static_cast<float*>(w.uT), Mp, Mp, stream));
  }
  const size_t eb = io_bytes(io);
  if (bf) {
    // dW_a and dW_x in one product over the 2D rows of dz^T (rows past D land in dW_x), so
    // the two share their rounds on the CUs and a last, partly filled round splits its K
    PlainGemmArgs q{};
    q.A = w.dzT_hi; q.A2 = w.dzT_lo; q.Bm = w.uT;
    q.M = 2 * D; q.N = D; q.K = Mp; q.lda = Mp; q.ldb = Mp; q.ldc = D;
    q.C = dW_a; q.C2 = dW_x; q.m_split = D; q.addend = nullptr;
    q.tail_ws = w.tail;
    RG_CHECK(launch_plain_gemm_bf16(q, stream));
  } else {
    for (int gi = 0; gi < 2; ++gi) {
      PlainGemmArgs q{};
      q.A = static_cast<const unsigned char*>(w.dzT_hi) + size_t(gi) * D * Mp * eb;
      q.A2 = nullptr;
      q.Bm = w.uT;
      q.M = D; q.N = D; q.K = Mp; q.lda = Mp; q.ldb = Mp; q.ldc = D;
      q.C = gi == 0 ? dW_a : dW_x;
      q.addend = nullptr;
      RG_CHECK(launch_plain_gemm_f32(q, stream));
    }
  }

  // 5. conv backward and the fixed-order reductions
  if (conv_w) {
    ConvBwdArgs cb{};
    cb.B = B; cb.T = T; cb.D = D; cb.x = x; cb.conv_w = conv_w; cb.conv_state = cs;
    cb.du = w.du; cb.dx = dx; cb.partial = w.conv_part;
    if (bf) RG_CHECK(launch_conv_bwd<bf16_t>(cb, stream));
    else RG_CHECK(launch_conv_bwd<float>(cb, stream));
  }
  ReduceArgs ra{};
  ra.D = D; ra.P = B * scan_chunks(T);
  ra.scan_part = w.scan_part; ra.conv_part = conv_w ? w.conv_part : nullptr;
  ra.lam = lambda; ra.c = c;
  ra.db_a = db_a; ra.db_x = db_x; ra.dlambda = dlambda;
  ra.dconv_w = dconv_w; ra.dconv_b = dconv_b;
  RG_CHECK(launch_reduce(ra, stream));
  return RGLRU_OK;
}

int rglru_bwd(int B, int T, int D, rglru_dtype io, float c, const void* x, const void* conv_w,
              const float* conv_b, const void* conv_state_in, const void* W_a, const void* W_x,
              const float* b_a, const float* b_x, const float* lambda, const float* h0,
              const void* dy, const float* dh_T, float* dx, float* dconv_w, float* dconv_b,
              float* dW_a, float* dW_x, float* db_a, float* db_x, float* dlambda, float* dh0,
              void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(kDefaultKnobs, B, T, D, io, c, x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a,
                  b_x, lambda, h0, dy, dh_T, dx, dconv_w, dconv_b, dW_a, dW_x, db_a, db_x, dlambda,
                  dh0, ws, ws_bytes, stream);
}

size_t rglru_train_saved_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_saved(cv, B, T, D, io);
  return cv.used;
}

size_t rglru_fwd_train_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_train(cv, B, T, D, io);
  return cv.used;
}

size_t rglru_bwd_saved_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (shape_status(B, T, D) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_bwd(cv, B, T, D, io, /*recompute=*/false);
  return cv.used;
}

int rglru_fwd_train(int B, int T, int D, rglru_dtype io, float c, const void* x,
                    const void* conv_w, const float* conv_b, const void* conv_state_in,
                    const void* W_a, const void* W_x, const float* b_a, const float* b_x,
                    const float* lambda, const float* h0, void* y, float* h_T,
                    void* conv_state_out, void* saved, size_t saved_bytes, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int st = shape_status(B, T, D);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !W_a || !W_x || !b_a || !b_x || !lambda || !y || !saved || !c_ok(c)) return RGLRU_EINVAL;
  for (const void* p : {x, conv_w, (const void*)conv_b, conv_state_in, W_a, W_x, (const void*)b_a,
                        (const void*)b_x, (const void*)lambda, (const void*)h0, (const void*)y,
                        (const void*)h_T, (const void*)conv_state_out, (const void*)saved,
                        (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (saved_bytes < rglru_train_saved_bytes(B, T, D, io)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_fwd_train_workspace_bytes(B, T, D, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  const TrainWs w = carve_train(cv, B, T, D, io);
  Carver sv(saved);
  const SavedAct a = carve_saved(sv, B, T, D, io);
  const void* u = nullptr;
  return forward_acts(io, B, T, D, c, x, conv_w, conv_b, conv_w ? conv_state_in : nullptr, W_a, W_x,
                      b_a, b_x, lambda, h0, a, w.tail, w.status, w.counter, y, h_T,
                      conv_state_out, kDefaultKnobs, stream, &u);
}

int rglru_bwd_saved(int B, int T, int D, rglru_dtype io, float c, const void* x,
                    const void* conv_w, const float* conv_b, const void* conv_state_in,
                    const void* W_a, const void* W_x, const float* lambda, const float* h0,
                    const void* dy, const float* dh_T, float* dx, float* dconv_w,
                    float* dconv_b, float* dW_a, float* dW_x, float* db_a, float* db_x,
                    float* dlambda, float* dh0, const void* saved, size_t saved_bytes, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (!saved) return RGLRU_EINVAL;
  return bwd_impl(kDefaultKnobs, B, T, D, io, c, x, conv_w, conv_b, conv_state_in, W_a, W_x,
                  nullptr, nullptr, lambda, h0, dy, dh_T, dx, dconv_w, dconv_b, dW_a, dW_x, db_a,
                  db_x, dlambda, dh0, ws, ws_bytes, stream, saved, saved_bytes);
}

size_t rglru_block_fwd_workspace_bytes(int B, int T, int D, int R, rglru_dtype io) {
  if (block_shape_status(B, T, D, R) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_block(cv, B, T, D, R, io);
  return cv.used;
}

static int block_impl(const Knobs& k, int B, int T, int D, int R, rglru_dtype io, float c,
                      const void* x, const void* W_in, const void* conv_w, const float* conv_b,
                      const void* conv_state_in, const void* W_a, const void* W_x,
                      const float* b_a, const float* b_x, const float* lambda, const float* h0,
                      const void* W_out, void* out, float* h_T, void* conv_state_out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  int st = block_shape_status(B, T, D, R);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !W_in || !W_a || !W_x || !b_a || !b_x || !lambda || !W_out || !out || !c_ok(c))
    return RGLRU_EINVAL;
  for (const void* p : {x, W_in, conv_w, (const void*)conv_b, conv_state_in, W_a, W_x,
                        (const void*)b_a, (const void*)b_x, (const void*)lambda, (const void*)h0,
                        W_out, (const void*)out, (const void*)h_T, (const void*)conv_state_out,
                        (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_block_fwd_workspace_bytes(B, T, D, R, io)) return RGLRU_EWORKSPACE;

  Carver cv(ws);
  BlockWs w = carve_block(cv, B, T, D, R, io);
  const int M = B * T;
  const bool bf = io == RGLRU_BF16;

  // 1. the two input linears: p and g = GeLU(.)
  if (bf) {
    BlockGemmArgs gi{};
    gi.A = x; gi.Bm = W_in; gi.M = M; gi.N = 2 * R; gi.K = D; gi.ldc = R;
    gi.C = w.p; gi.G = w.g; gi.split = R;
    RG_CHECK(launch_block_gemm_bf16(gi, stream));
  } else {
    PlainGemmArgs pa{};
    pa.A = x; pa.Bm = W_in; pa.M = M; pa.N = 2 * R; pa.K = D;
    pa.lda = D; pa.ldb = D; pa.ldc = 2 * R; pa.C = w.pq;
    RG_CHECK(launch_plain_gemm_f32(pa, stream));
    RG_CHECK(launch_split_gelu_f32(w.pq, M, R, static_cast<float*>(w.p), static_cast<float*>(w.g), stream));
  }

  // 2. the temporal branch on p (the conv launch also initialises the look-back status)
  const void* u = w.p;
  bool prefilled = false;
  if (conv_w) {
    uint32_t* fill = static_cast<uint32_t*>(w.lru.status);
    const size_t words = status_fill_words(B, T, R, io, /*fused=*/true);
    if (bf)
      RG_CHECK(launch_conv_fwd<bf16_t>(B, T, R, w.p, conv_w, conv_b, conv_state_in, w.lru.u,
                                       conv_state_out, stream, fill, words, w.lru.counter));
    else
      RG_CHECK(launch_conv_fwd<float>(B, T, R, w.p, conv_w, conv_b, conv_state_in, w.lru.u,
                                      conv_state_out, stream, fill, words, w.lru.counter));
    u = w.lru.u;
    prefilled = true;
  }
  if (bf) {
    // the fused layer multiplies by g before rounding: z = RNE(h g).  z goes over p once
    // the conv has consumed it; without the conv p is the layer's input, whose rows every
    // channel tile reads, so z goes to the (then unused) u buffer.
    w.y = conv_w ? w.p : w.lru.u;
    LruArgs la{};
    la.u = u; la.Wa = W_a; la.Wx = W_x; la.ba = b_a; la.bx = b_x; la.lam = lambda; la.c = c;
    la.h0 = h0; la.y = w.y; la.hT = h_T; la.gate = w.g; la.B = B; la.T = T; la.D = R;
    la.status = static_cast<uint32_t*>(w.lru.status); la.counters = w.lru.counter;
    la.ticket_guess = k.lru_ticket_guess; la.max_polls = k.lookback_polls;
    la.stall = w.lru.counter + kStallWord;
    RG_CHECK(launch_lru_fused(la, prefilled, stream));
  } else {
    st = lru_layer(io, B, T, R, c, u, W_a, W_x, b_a, b_x, lambda, h0, w.y, h_T, w.lru, prefilled,
                   k, stream);
    if (st != RGLRU_OK) return st;
    RG_CHECK(launch_mul_f32(static_cast<float*>(w.y), static_cast<const float*>(w.g), size_t(M) * R,
                            stream));
  }

  // 3. the output linear on z
  if (bf) {
    BlockGemmArgs go{};
    go.A = w.y; go.Bm = W_out; go.M = M; go.N = D; go.K = R; go.ldc = D;
    go.C = out; go.G = nullptr; go.split = 0; go.tail_ws = w.tail;
    RG_CHECK(launch_block_gemm_bf16(go, stream));
  } else {
    PlainGemmArgs po{};
    po.A = w.y; po.Bm = W_out; po.M = M; po.N = D; po.K = R;
    po.lda = R; po.ldb = R; po.ldc = D; po.C = static_cast<float*>(out);
    RG_CHECK(launch_plain_gemm_f32(po, stream));
  }
  return RGLRU_OK;
}

int rglru_block_fwd(int B, int T, int D, int R, rglru_dtype io, float c, const void* x,
                    const void* W_in, const void* conv_w, const float* conv_b,
                    const void* conv_state_in, const void* W_a, const void* W_x,
                    const float* b_a, const float* b_x, const float* lambda, const float* h0,
                    const void* W_out, void* out, float* h_T, void* conv_state_out, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  return block_impl(kDefaultKnobs, B, T, D, R, io, c, x, W_in, conv_w, conv_b, conv_state_in, W_a,
                    W_x, b_a, b_x, lambda, h0, W_out, out, h_T, conv_state_out, ws, ws_bytes,
                    stream);
}

int rglru_workspace_status(const void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned16(ws)) return RGLRU_EINVAL;
  if (ws_bytes < kCounterWords * sizeof(uint32_t)) return RGLRU_EWORKSPACE;
  uint32_t flag = 0;
  RG_CHECK(hipMemcpyAsync(&flag, static_cast<const uint32_t*>(ws) + kStallWord, sizeof(flag),
                          hipMemcpyDeviceToHost, stream));
  RG_CHECK(hipStreamSynchronize(stream));
  return flag ? RGLRU_ESTALL : RGLRU_OK;
}

size_t gated_mlp_fwd_workspace_bytes(int B, int T, int D, int MD, rglru_dtype io) {
  if (mlp_shape_status(B, T, D, MD) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_mlp(cv, B, T, D, MD, io);
  return cv.used;
}

int gated_mlp_fwd(int B, int T, int D, int MD, rglru_dtype io, const void* x, const void* W_1,
                  const void* W_2, const void* W_3, void* out, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  int st = mlp_shape_status(B, T, D, MD);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !W_1 || !W_2 || !W_3 || !out) return RGLRU_EINVAL;
  for (const void* p : {x, W_1, W_2, W_3, (const void*)out, (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < gated_mlp_fwd_workspace_bytes(B, T, D, MD, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  MlpWs w = carve_mlp(cv, B, T, D, MD, io);
  const int M = B * T;
  if (io == RGLRU_BF16) {
    GegluGemmArgs g1{};
    g1.A = x; g1.W1 = W_1; g1.W2 = W_2; g1.M = M; g1.N = MD; g1.K = D; g1.H = w.h;
    RG_CHECK(launch_geglu_gemm_bf16(g1, stream));
    BlockGemmArgs g3{};
    g3.A = w.h; g3.Bm = W_3; g3.M = M; g3.N = D; g3.K = MD; g3.ldc = D;
    g3.C = out; g3.G = nullptr; g3.split = 0; g3.tail_ws = w.tail;
    RG_CHECK(launch_block_gemm_bf16(g3, stream));
    return RGLRU_OK;
  }
  float* q1 = static_cast<float*>(w.h);
  PlainGemmArgs pa{};
  pa.A = x; pa.Bm = W_1; pa.M = M; pa.N = MD; pa.K = D; pa.lda = D; pa.ldb = D; pa.ldc = MD;
  pa.C = q1;
  RG_CHECK(launch_plain_gemm_f32(pa, stream));
  pa.Bm = W_2; pa.C = w.q2;
  RG_CHECK(launch_plain_gemm_f32(pa, stream));
  RG_CHECK(launch_geglu_f32(q1, w.q2, q1, size_t(M) * MD, stream));
  PlainGemmArgs po{};
  po.A = q1; po.Bm = W_3; po.M = M; po.N = D; po.K = MD; po.lda = MD; po.ldb = MD; po.ldc = D;
  po.C = static_cast<float*>(out);
  RG_CHECK(launch_plain_gemm_f32(po, stream));
  return RGLRU_OK;
}

size_t local_mqa_fwd_workspace_bytes(int B, int T, int D, rglru_dtype io) {
  if (mqa_shape_status(B, T, D, 1, 0) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  carve_mqa(cv, B, T, D, io);
  return cv.used;
}

int local_mqa_fwd(int B, int T, int D, rglru_dtype io, int window, int pos0, const void* x,
                  const void* W_qkv, const void* W_o, void* out, void* k_out, void* v_out,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = mqa_shape_status(B, T, D, window, pos0);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x || !W_qkv || !W_o || !out) return RGLRU_EINVAL;
  for (const void* p : {x, W_qkv, W_o, (const void*)out, (const void*)k_out, (const void*)v_out,
                        (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < local_mqa_fwd_workspace_bytes(B, T, D, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  MqaWs w = carve_mqa(cv, B, T, D, io);
  if (k_out) w.k = k_out;
  if (v_out) w.v = v_out;
  const int M = B * T;
  const bool bf = io == RGLRU_BF16;
  if (bf) {
    QkvGemmArgs g{};
    g.A = x; g.W = W_qkv; g.M = M; g.D = D; g.T = T; g.pos0 = pos0;
    g.q = w.q; g.k = w.k; g.v = w.v;
    RG_CHECK(launch_qkv_gemm_bf16(g, stream));
  } else {
    const float* W = static_cast<const float*>(W_qkv);
    PlainGemmArgs pa{};
    pa.A = x; pa.M = M; pa.K = D; pa.lda = D; pa.ldb = D;
    pa.Bm = W; pa.N = D; pa.ldc = D; pa.C = static_cast<float*>(w.q);
    RG_CHECK(launch_plain_gemm_f32(pa, stream));
    pa.Bm = W + size_t(D) * D; pa.N = kHeadDim; pa.ldc = kHeadDim; pa.C = static_cast<float*>(w.k);
    RG_CHECK(launch_plain_gemm_f32(pa, stream));
    pa.Bm = W + size_t(D + kHeadDim) * D; pa.C = static_cast<float*>(w.v);
    RG_CHECK(launch_plain_gemm_f32(pa, stream));
    RG_CHECK(launch_rope_f32(static_cast<float*>(w.q), M, D, T, pos0, stream));
    RG_CHECK(launch_rope_f32(static_cast<float*>(w.k), M, kHeadDim, T, pos0, stream));
  }
  MqaArgs a{};
  a.q = w.q; a.k = w.k; a.v = w.v; a.o = w.attn;
  a.B = B; a.T = T; a.S = T; a.H = D / kHeadDim;
  a.window = window; a.q_pos0 = pos0; a.kv_pos0 = pos0;
  a.scale_log2 = float(1.4426950408889634 / sqrt(double(kHeadDim)));
  RG_CHECK(launch_mqa_fwd(a, bf, stream));
  if (bf) {
    BlockGemmArgs go{};
    go.A = w.attn; go.Bm = W_o; go.M = M; go.N = D; go.K = D; go.ldc = D;
    go.C = out; go.G = nullptr; go.split = 0; go.tail_ws = w.tail;
    RG_CHECK(launch_block_gemm_bf16(go, stream));
  } else {
    PlainGemmArgs po{};
    po.A = w.attn; po.Bm = W_o; po.M = M; po.N = D; po.K = D; po.lda = D; po.ldb = D; po.ldc = D;
    po.C = static_cast<float*>(out);
    RG_CHECK(launch_plain_gemm_f32(po, stream));
  }
  return RGLRU_OK;
}

size_t local_mqa_decode_workspace_bytes(int B, int D, rglru_dtype io) {
  if (mqa_shape_status(B, 1, D, 1, 0) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  const size_t n = size_t(B) * D * io_bytes(io);
  cv.take<unsigned char>(io == RGLRU_BF16 ? mqa_decode_partial_bytes(B, D)
                                          : size_t(B) * (D + 2 * kHeadDim) * sizeof(float));
  cv.take<unsigned char>(n);
  cv.take<unsigned char>(n);
  return cv.used;
}

int local_mqa_decode_step(int B, int D, rglru_dtype io, int window, const int* pos, const void* x_t,
                          const void* W_qkv, const void* W_o, void* k_cache, void* v_cache,
                          void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = mqa_shape_status(B, 1, D, window, 0);
  if (st != RGLRU_OK) return st;
  if (int64_t(B) * window * kHeadDim >= (int64_t(1) << 31)) return RGLRU_ESHAPE;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!pos || !x_t || !W_qkv || !W_o || !k_cache || !v_cache || !out) return RGLRU_EINVAL;
  for (const void* p : {(const void*)pos, x_t, W_qkv, W_o, (const void*)k_cache, (const void*)v_cache,
                        (const void*)out, (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < local_mqa_decode_workspace_bytes(B, D, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  const size_t n = size_t(B) * D * io_bytes(io);
  MqaDecodeArgs a{};
  a.bf16 = io == RGLRU_BF16;
  a.B = B; a.D = D; a.window = window; a.pos = pos;
  a.x = x_t; a.Wqkv = W_qkv; a.Wo = W_o; a.kcache = k_cache; a.vcache = v_cache; a.out = out;
  a.partial = reinterpret_cast<float*>(cv.take<unsigned char>(
      a.bf16 ? mqa_decode_partial_bytes(B, D) : size_t(B) * (D + 2 * kHeadDim) * sizeof(float)));
  a.qbuf = cv.take<unsigned char>(n);
  a.attn = cv.take<unsigned char>(n);
  RG_CHECK(launch_mqa_decode(a, stream));
  return RGLRU_OK;
}

size_t rglru_block_decode_workspace_bytes(int B, int D, int R, rglru_dtype io) {
  if (block_shape_status(B, 1, D, R) != RGLRU_OK || !io_ok(io)) return 0;
  Carver cv(nullptr);
  const size_t n = size_t(B) * R;
  if (io == RGLRU_BF16) {
    const size_t a = splitk_partial_bytes(B, 2 * R, D), b = splitk_partial_bytes(B, D, R);
    cv.take<unsigned char>(a > b ? a : b);          // split-K partials of both linears
    cv.take<unsigned char>(decode_partial_bytes(B, R));
  } else {
    cv.take<float>(2 * n);                          // the input linears' product
  }
  for (int i = 0; i < 4; ++i) cv.take<unsigned char>(n * io_bytes(io));   // p, g, u, z
  return cv.used;
}

int rglru_block_decode_step(int B, int D, int R, rglru_dtype io, float c, const void* x_t,
                            const void* W_in, const void* conv_w, const float* conv_b,
                            void* conv_state, const void* W_a, const void* W_x, const float* b_a,
                            const float* b_x, const float* lambda, float* h, const void* W_out,
                            void* out_t, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = block_shape_status(B, 1, D, R);
  if (st != RGLRU_OK) return st;
  if (!io_ok(io)) return RGLRU_EDTYPE;
  if (!x_t || !W_in || !W_a || !W_x || !b_a || !b_x || !lambda || !h || !W_out || !out_t || !c_ok(c))
    return RGLRU_EINVAL;
  if (conv_w && !conv_state) return RGLRU_EINVAL;
  for (const void* p : {x_t, W_in, conv_w, (const void*)conv_b, (const void*)conv_state, W_a, W_x,
                        (const void*)b_a, (const void*)b_x, (const void*)lambda, (const void*)h, W_out,
                        (const void*)out_t, (const void*)ws})
    if (p && !aligned16(p)) return RGLRU_EINVAL;
  if (!ws || ws_bytes < rglru_block_decode_workspace_bytes(B, D, R, io)) return RGLRU_EWORKSPACE;
  Carver cv(ws);
  const size_t n = size_t(B) * R;
  const bool bf = io == RGLRU_BF16;
  float* part = nullptr;
  float* dpart = nullptr;
  float* pq = nullptr;
  if (bf) {
    const size_t a = splitk_partial_bytes(B, 2 * R, D), b = splitk_partial_bytes(B, D, R);
    part = reinterpret_cast<float*>(cv.take<unsigned char>(a > b ? a : b));
    dpart = reinterpret_cast<float*>(cv.take<unsigned char>(decode_partial_bytes(B, R)));
  } else {
    pq = cv.take<float>(2 * n);
  }
  void* p = cv.take<unsigned char>(n * io_bytes(io));
  void* g = cv.take<unsigned char>(n * io_bytes(io));
  void* u = cv.take<unsigned char>(n * io_bytes(io));
  void* z = cv.take<unsigned char>(n * io_bytes(io));

  // 1. the input linears: p and g = GeLU(.)
  if (bf) {
    const int S = splitk_splits(B, 2 * R, D);
    RG_CHECK(launch_splitk_bf16(x_t, W_in, B, 2 * R, D, S, part, stream));
    RG_CHECK(launch_splitk_inproj_bf16(part, S, B, R, p, g, stream));
  } else {
    PlainGemmArgs pa{};
    pa.A = x_t; pa.Bm = W_in; pa.M = B; pa.N = 2 * R; pa.K = D; pa.lda = D; pa.ldb = D; pa.ldc = 2 * R;
    pa.C = pq;
    RG_CHECK(launch_plain_gemm_f32(pa, stream));
    RG_CHECK(launch_split_gelu_f32(pq, B, R, static_cast<float*>(p), static_cast<float*>(g), stream));
  }
  // 2. the branch's decode step on p, the state (h, conv history) updated in place
  const void* uin = p;
  if (conv_w) {
    if (bf) RG_CHECK(launch_conv_decode<bf16_t>(B, R, p, conv_w, conv_b, conv_state, u, stream));
    else RG_CHECK(launch_conv_decode<float>(B, R, p, conv_w, conv_b, conv_state, u, stream));
    uin = u;
  }
  if (bf) {
    DecodeArgs d{};
    d.u = uin; d.Wa = W_a; d.Wx = W_x; d.ba = b_a; d.bx = b_x; d.lam = lambda; d.c = c;
    d.h = h; d.y = z; d.partial = dpart; d.B = B; d.D = R; d.gate = g;
    RG_CHECK(launch_decode_bf16(d, stream));
  } else {
    GateGemmArgs ga{};
    ga.U = uin; ga.Wa = W_a; ga.Wx = W_x; ga.M = B; ga.N = R; ga.K = R;
    ga.ba = b_a; ga.bx = b_x; ga.lam = lambda; ga.c = c;
    ga.u = uin; ga.h = h; ga.y = z;
    st = gate_projection(io, ga, kEpiDecode, pq, pq + n, stream);
    if (st != RGLRU_OK) return st;
    RG_CHECK(launch_mul_f32(static_cast<float*>(z), static_cast<const float*>(g), n, stream));
  }
  // 3. the output linear on z
  if (bf) {
    const int S = splitk_splits(B, D, R);
    RG_CHECK(launch_splitk_bf16(z, W_out, B, D, R, S, part, stream));
    RG_CHECK(launch_splitk_out_bf16(part, S, B, D, out_t, stream));
  } else {
    PlainGemmArgs po{};
    po.A = z; po.Bm = W_out; po.M = B; po.N = D; po.K = R; po.lda = R; po.ldb = R; po.ldc = D;
    po.C = static_cast<float*>(out_t);
    RG_CHECK(launch_plain_gemm_f32(po, stream));
  }
  return RGLRU_OK;
}

// ------------------------------------------------------------------ test entry points
// Declared in rglru_testing.h (not part of the public header): the public calls with the
// chained-scan settings passed explicitly instead of kDefaultKnobs.

static Knobs knobs_of(const rglru_testing_knobs* t) {
  return t ? Knobs{t->lru_ticket_guess, t->scan_direct_polls, t->lookback_polls, t->lru_force_fused}
           : kDefaultKnobs;
}

void rglru_testing_default_knobs(rglru_testing_knobs* t) {
  if (!t) return;
  t->lru_ticket_guess = kDefaultKnobs.lru_ticket_guess;
  t->scan_direct_polls = kDefaultKnobs.scan_direct_polls;
  t->lookback_polls = kDefaultKnobs.lookback_polls;
  t->lru_force_fused = kDefaultKnobs.lru_force_fused;
}

int rglru_testing_fwd(const rglru_testing_knobs* t, int B, int T, int D, rglru_dtype io, float c,
                      const void* x, const void* conv_w, const float* conv_b,
                      const void* conv_state_in, const void* W_a, const void* W_x,
                      const float* b_a, const float* b_x, const float* lambda, const float* h0,
                      void* y, float* h_T, void* conv_state_out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  return fwd_impl(knobs_of(t), B, T, D, io, c, x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a,
                  b_x, lambda, h0, y, h_T, conv_state_out, ws, ws_bytes, stream);
}

int rglru_testing_scan(const rglru_testing_knobs* t, int B, int T, int D, rglru_dtype io,
                       const void* x, const void* conv_w, const float* conv_b,
                       const void* conv_state_in, const float* a, const float* beta,
                       const float* h0, void* y, float* h_T, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return scan_impl(knobs_of(t), B, T, D, io, x, conv_w, conv_b, conv_state_in, a, beta, h0, y,
                   h_T, ws, ws_bytes, stream);
}

int rglru_testing_bwd(const rglru_testing_knobs* t, int B, int T, int D, rglru_dtype io, float c,
                      const void* x, const void* conv_w, const float* conv_b,
                      const void* conv_state_in, const void* W_a, const void* W_x,
                      const float* b_a, const float* b_x, const float* lambda, const float* h0,
                      const void* dy, const float* dh_T, float* dx, float* dconv_w,
                      float* dconv_b, float* dW_a, float* dW_x, float* db_a, float* db_x,
                      float* dlambda, float* dh0, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(knobs_of(t), B, T, D, io, c, x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a,
                  b_x, lambda, h0, dy, dh_T, dx, dconv_w, dconv_b, dW_a, dW_x, db_a, db_x, dlambda,
                  dh0, ws, ws_bytes, stream);
}

int rglru_testing_block_fwd(const rglru_testing_knobs* t, int B, int T, int D, int R,
                            rglru_dtype io, float c, const void* x, const void* W_in,
                            const void* conv_w, const float* conv_b, const void* conv_state_in,
                            const void* W_a, const void* W_x, const float* b_a, const float* b_x,
                            const float* lambda, const float* h0, const void* W_out, void* out,
                            float* h_T, void* conv_state_out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return block_impl(knobs_of(t), B, T, D, R, io, c, x, W_in, conv_w, conv_b, conv_state_in, W_a,
                    W_x, b_a, b_x, lambda, h0, W_out, out, h_T, conv_state_out, ws, ws_bytes,
                    stream);
}

}  // extern "C"
