// Host-side launchers of the gfx950 kernels (internal to librglru.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rglru {

// ---------------------------------------------------------------- chained-scan settings
// Every workspace of a call that runs a chained scan starts with 64 counter words, zeroed
// by the call: ticket counters, and at kStallWord the flag a look-back sets when it gives up
// waiting for a predecessor chunk (rglru_workspace_status reads it).
constexpr int kCounterWords = 64;
constexpr int kStallWord = 63;
// Polls of an unpublished predecessor before the forward scan computes its summary itself.
constexpr int kDirectPolls = 2048;
// Settings of the chained scans that only the test entry points change; every public entry
// point runs with kDefaultKnobs.
struct Knobs {
  int lru_ticket_guess;   // fused RG-LRU kernel: shift of the launch-order ticket guess
  int scan_direct_polls;  // forward scan: see ScanFwdArgs::direct_polls
  int lookback_polls;     // fused kernel and reverse scan: polls before a look-back gives up
  int lru_force_fused;    // bf16 RG-LRU layer: the fused kernel whatever the shape (1) or by shape (0)
};
extern const Knobs kDefaultKnobs;

// ---------------------------------------------------------------- conv.hip
// With fill/counter, the same launch also prepares the look-back status of a following
// scan (fill_words words set to all ones, counter[0..63] = 0).
template <typename IO>
hipError_t launch_conv_fwd(int B, int T, int D, const void* x, const void* w, const float* cb,
                           const void* state_in, void* u, void* state_out, hipStream_t s,
                           uint32_t* fill = nullptr, size_t fill_words = 0,
                           uint32_t* counter = nullptr);
template <typename IO>
hipError_t launch_conv_decode(int B, int D, const void* x, const void* w, const float* cb,
                              void* hist, void* u, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
// status[0..words) = all ones, counters[0..ncounters) = 0 (ncounters <= 256), one launch
hipError_t launch_fill_status(uint32_t* status, size_t words, uint32_t* counters, int ncounters,
                              hipStream_t s);

// ---------------------------------------------------------------- gemm.hip
// Epilogue kinds of the gate projection z = U [W_a; W_x]^T (Eq. (1)-(2)).
enum GateEpi : int {
  kEpiAB = 0,      // write a, beta = m i           (forward)
  kEpiRI = 1,      // write r, i                    (backward recompute)
  kEpiDecode = 2,  // h <- a h + beta u, y = RNE(h) (fp32 decode step)
};

struct GateGemmArgs {
  const void* U;      // [M, K] io, row stride K
  const void* Wa;     // [N, K] io
  const void* Wx;     // [N, K] io
  int M, N, K;        // N = K = D
  const float* ba;
  const float* bx;
  const float* lam;
  float c;
  float* out0;        // kEpiAB: a  ; kEpiRI: r  [M, N]
  float* out1;        // kEpiAB: beta; kEpiRI: i [M, N]
  const void* u;      // kEpiDecode: u [M, N] io
  float* h;           // kEpiDecode: state [M, N] in/out
  void* y;            // kEpiDecode: y [M, N] io
  // bf16 kEpiAB / kEpiRI: fp32 partials (gate_gemm_tail_bytes bytes) or NULL; with them the
  // tiles of a last, partly filled round split their K loop and a fixup applies the gates
  float* tail_ws;
};
size_t gate_gemm_tail_bytes(int M, int N, int K);

// One bf16 decode step after the conv: split-K gate projection into `partial`, then the
// fixed-order sum, the gates and the state update (decode.hip).
struct DecodeArgs {
  const void* u;      // [B, D] bf16, the conv output of the step
  const void* Wa;     // [D, D] bf16
  const void* Wx;     // [D, D] bf16
  const float* ba;
  const float* bx;
  const float* lam;
  float c;
  float* h;           // [B, D] state, in/out
  void* y;            // [B, D] bf16
  float* partial;     // decode_partial_bytes(B, D): the split sums, then 3 D gate constants
  int B, D;
  int splits;         // set by the launcher
  float* chan;        // set by the launcher: [3, D] per-channel gate constants
  const void* gate;   // [B, D] bf16 or NULL: y = RNE(h * gate) instead of RNE(h)
};
int decode_splits(int B, int D);
size_t decode_partial_bytes(int B, int D);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

// C[M,N] = A[M,K] B[N,K]^T (+ addend), fp32 output.  With A2 (bf16 only) the product
// is (A + A2) B^T, evaluated as two bf16 MFMA passes over K.
struct PlainGemmArgs {
  const void* A;
  const void* A2;
  const void* Bm;
  int M, N, K;
  int lda, ldb, ldc;
  float* C;
  const float* addend;   // may equal C (read before write by the same thread) or NULL
  // bf16 operands only: rows m >= m_split go to C2 (row m - m_split, same ldc; addend must
  // be NULL then); m_split = 0 means M (everything in C).  tail_ws (plain_gemm_tail_bytes
  // bytes, or NULL) lets the tiles of a last, partly filled round split their K loop.
  float* C2;
  int m_split;
  float* tail_ws;
};
// fp32 partials a plain bf16 GEMM of this shape needs for its split tail (0: no split).
size_t plain_gemm_tail_bytes(int M, int N, int K);

// The linears of the recurrent block, bf16 in and out, C = A Bm^T with row strides K.
// With G: N = 2 split columns, C[M, split] = the first split columns, G[M, split] = GeLU of
// the rest (ldc = split); without G: C[M, N] (ldc = N).
// Without G, tail_ws (out_gemm_tail_bytes(M, N, K) bytes, or NULL) lets the tiles of a last,
// partly filled round split their K loop (fp32 partials, then a fixed-order fixup).
struct BlockGemmArgs {
  const void* A;
  const void* Bm;
  int M, N, K;
  int ldc;
  void* C;
  void* G;
  int split;
  float* tail_ws;
};
hipError_t launch_block_gemm_bf16(const BlockGemmArgs& g, hipStream_t s);
size_t out_gemm_tail_bytes(int M, int N, int K);

// First layer of the gated MLP block, bf16: H[M, N] = RNE(GeLU(A W1^T) * (A W2^T)) with
// A [M, K], W1, W2 [N, K] (row strides K, N).
struct GegluGemmArgs {
  const void* A;
  const void* W1;
  const void* W2;
  int M, N, K;
  void* H;
};
hipError_t launch_geglu_gemm_bf16(const GegluGemmArgs& g, hipStream_t s);

// Projections of the local-MQA block, bf16: [q k v] = A [W_q; W_k; W_v]^T with W [D + 256, D],
// q [M, D] and k [M, 128] rotated by RoPE at position pos0 + m % T, v [M, 128].
struct QkvGemmArgs {
  const void* A;
  const void* W;
  int M, D, T, pos0;
  void* q;
  void* k;
  void* v;
};
hipError_t launch_qkv_gemm_bf16(const QkvGemmArgs& g, hipStream_t s);

hipError_t launch_gate_gemm_bf16(const GateGemmArgs& g, int epi, hipStream_t s);   // kEpiAB, kEpiRI
hipError_t launch_plain_gemm_bf16(const PlainGemmArgs& g, hipStream_t s);
hipError_t launch_plain_gemm_f32(const PlainGemmArgs& g, hipStream_t s);
// C0 = A B0^T and C1 = A B1^T (fp32, [M,N], K-contiguous operands) in one launch
hipError_t launch_gemm_f32_pair(const float* A, const float* B0, const float* B1, int M, int N,
                                int K, float* C0, float* C1, hipStream_t s);
// fp32 I/O: gate math from pre-activations za, zx [M, N] (already W u, bias not added).
hipError_t launch_gate_elementwise_f32(const GateGemmArgs& g, const float* za, const float* zx,
                                       int epi, hipStream_t s);

// ---------------------------------------------------------------- block.hip
// fp32 I/O steps of the recurrent block: pq [M, 2R] -> p = pq[:, :R], g = GeLU(pq[:, R:]);
// y *= g elementwise.
hipError_t launch_split_gelu_f32(const float* pq, int M, int R, float* p, float* g, hipStream_t s);
hipError_t launch_mul_f32(float* y, const float* g, size_t n, hipStream_t s);
// h[i] = RNE_f32(GeLU(q1[i]) * q2[i]) (GeLU in fp64): the gated MLP's product for fp32 I/O
hipError_t launch_geglu_f32(const float* q1, const float* q2, float* h, size_t n, hipStream_t s);

// ---------------------------------------------------------------- mqa.hip
// Sliding-window multi-query attention over rotated q [B,T,H,128], k, v [B,S,128] (io
// dtype); query t is at absolute position q_pos0 + t, key s at kv_pos0 + s.
struct MqaArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;                // [B,T,H,128]
  int B, T, S, H;
  int window;
  int q_pos0, kv_pos0;
  float scale_log2;       // log2(e) / sqrt(128)
};
hipError_t launch_mqa_fwd(const MqaArgs& a, bool bf16, hipStream_t s);
// x [M, ncols] fp32 in place: RoPE on every 128-wide head vector, row m at position
// pos0 + m % T (fp64 angles)
hipError_t launch_rope_f32(float* x, int M, int ncols, int T, int pos0, hipStream_t s);

// ---------------------------------------------------------------- mqa_decode.hip
// One local-MQA generation step with a bounded cache (k, v caches [B, W, 128], slot
// pos % W); x [B, D], W_qkv [D + 256, D], W_o [D, D]; pos [B] int32 on the device.
struct MqaDecodeArgs {
  bool bf16;
  int B, D, window;
  const int* pos;
  const void* x;
  const void* Wqkv;
  const void* Wo;
  void* kcache;
  void* vcache;
  void* out;             // [B, D]
  float* partial;        // mqa_decode_partial_bytes(B, D)
  void* qbuf;            // [B, D] io
  void* attn;            // [B, D] io
};
size_t mqa_decode_partial_bytes(int B, int D);
hipError_t launch_mqa_decode(const MqaDecodeArgs& a, hipStream_t s);
// Small-M bf16 products for decode steps: partial[S][M][N] = the S K-range partial sums of
// A [M,K] Bm [N,K]^T (S = splitk_splits(M, N, K)), then RNE_bf16 of their fixed-order sum.
int splitk_splits(int M, int N, int K);
size_t splitk_partial_bytes(int M, int N, int K);
hipError_t launch_splitk_bf16(const void* A, const void* Bm, int M, int N, int K, int S, float* partial,
                             hipStream_t s);
hipError_t launch_splitk_out_bf16(const float* partial, int S, int M, int N, void* out, hipStream_t s);
// The recurrent block's input linears in a decode step: p = RNE(sum), g = RNE(GeLU(sum)) of
// the partial sums [S][M][2R] (columns [0, R) and [R, 2R)).
hipError_t launch_splitk_inproj_bf16(const float* partial, int S, int M, int R, void* p, void* g,
                                     hipStream_t s);

// ---------------------------------------------------------------- lru.hip
// The fused RG-LRU layer (gate GEMM + log-space gates + chunked scan) for bf16 I/O.
struct LruArgs {
  const void* u;          // [B,T,D] bf16 (the conv output)
  const void* Wa;
  const void* Wx;
  const float* ba;
  const float* bx;
  const float* lam;
  float c;
  const float* h0;        // [B,D] or NULL
  void* y;                // [B,T,D] bf16: RNE(h), or RNE(h * gate) with a gate
  float* hT;              // [B,D] or NULL
  int B, T, D;
  uint32_t* status;       // lru_status_bytes(B,T,D) bytes of look-back words
  uint32_t* counters;     // 64 ticket counters (zeroed with the status words)
  int groups;             // set by the launcher
  int chain_bw;           // sequences per block of the chain order (set by the launcher)
  const void* gate;       // [B,T,D] bf16 multiplier of the output (the block's GeLU branch) or NULL
  int ticket_guess;       // added to the launch-order ticket guess (0; tests shift it)
  int max_polls;          // look-back polls before giving up (kMaxPolls; < 0: at once)
  uint32_t* stall;        // set to 1 when a look-back gives up (counters + kStallWord)
};
int lru_chunks(int T);
long lru_tiles(int B, int T, int D);   // workgroups of one fused launch
size_t lru_status_bytes(int B, int T, int D);
hipError_t launch_lru_fused(const LruArgs& a, bool prefilled, hipStream_t s);

// ---------------------------------------------------------------- scan.hip
struct ScanFwdArgs {
  int B, T, D;
  const void* x;          // [B,T,D] io (conv input, or u itself when conv_w is NULL)
  const void* conv_w;     // [4,D] io or NULL
  const float* conv_b;
  const void* conv_state; // [B,3,D] io or NULL
  const float* a;         // [B,T,D] fp32   (kEpiAB layout) -- or r when from_ri
  const float* beta;      // [B,T,D] fp32                   -- or i when from_ri
  bool from_ri;           // gates given as (r, i): a, beta recomputed with lam, c
  bool from_z;            // gates given as the projections (z^a, z^x): r = sigma(z^a + zb_a),
                          // i = sigma(z^x + zb_x), then as from_ri
  const float* zb_a;      // [D] biases of the from_z mode
  const float* zb_x;
  const float* lam;
  float c;
  const float* h0;        // [B,D] or NULL
  void* y;                // [B,T,D] io or NULL
  void* h_all;            // [B,T,D] of the scan state type (Acc), or NULL: every h_t
  float* h_T;             // [B,D] or NULL
  void* status;           // look-back words, scan_status_bytes(B,T,D,sizeof(Acc)) bytes
  uint32_t* counter;      // 64 words zeroed with the status words (the forward scan takes no tickets)
  bool prefilled;         // status and counters already initialised on this stream
  int groups;             // tile groups, set by the launcher
  int direct_polls;       // look-back polls of an unpublished predecessor before its summary
                          // is computed from memory (kDirectPolls; < 0: always, ignoring
                          // published values)
};
// Look-back status bytes of a scan whose state type has acc_bytes bytes (4 or 8).
size_t scan_status_bytes(int B, int T, int D, int acc_bytes);
long scan_fwd_tiles(int B, int T, int D);   // workgroups of one forward scan launch
// Acc = float for bf16 I/O, double for fp32 I/O.
template <typename IO, typename Acc> hipError_t launch_scan_fwd(const ScanFwdArgs& a, hipStream_t s);

struct ScanBwdArgs {
  int B, T, D;
  const void* u;          // [B,T,D] io
  const float* r;         // [B,T,D] fp32
  const float* i;         // [B,T,D] fp32
  const void* h_all;      // [B,T,D] of the scan state type (Acc), h_t
  const float* h0;        // [B,D] or NULL
  const void* dy;         // [B,T,D] io
  const float* dh_T;      // [B,D] or NULL
  const float* lam;
  float c;
  // outputs
  void* dz_hi;            // [B*T, 2D]: bf16 hi part (bf16 io) or fp32 dz (fp32 io)
  void* dz_lo;            // [B*T, 2D] bf16 lo part (bf16 io only)
  float* du;              // [B,T,D] fp32: G m i (the direct term of du)
  float* dh0;             // [B,D] or NULL
  double* partial;        // [B * nchunks, 3, D]: db_a, db_x, dL partial sums
  void* status;
  uint32_t* counter;      // 64 words: the ticket counter, ..., the stall flag (kStallWord)
  int max_polls;          // look-back polls before giving up (kMaxPolls; < 0: at once)
  uint32_t* stall;        // set to 1 when a look-back gives up
};
int scan_chunks(int T);
template <typename IO, typename Acc> hipError_t launch_scan_bwd(const ScanBwdArgs& a, hipStream_t s);

// ---------------------------------------------------------------- bwd.hip
template <typename E>
hipError_t launch_transpose(const E* src, int R, int C, int lds_src, E* dst, int ldd, int Rp,
                            hipStream_t s);
struct ConvBwdArgs {
  int B, T, D;
  const void* x;
  const void* conv_w;
  const void* conv_state;
  const float* du;       // [B,T,D]
  float* dx;             // [B,T,D]
  double* partial;       // [B * nchunks, 5, D]: dconv_w[0..3], dconv_b partial sums
};
template <typename IO> hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t s);
struct ReduceArgs {
  int D;
  int P;                   // number of partial rows per quantity
  const double* scan_part;  // [P, 3, D]
  const double* conv_part;  // [P, 5, D] or NULL
  const float* lam;
  float c;
  float* db_a;
  float* db_x;
  float* dlambda;
  float* dconv_w;          // [4, D] or NULL
  float* dconv_b;          // [D] or NULL
};
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);

}  // namespace rglru
