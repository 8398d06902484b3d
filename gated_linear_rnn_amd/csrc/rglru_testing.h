/*
 * rglru_testing.h - test-only entry points of librglru.so (not part of the public interface
 * in include/rglru.h).
 *
 * The chained scans of the library (the fused RG-LRU kernel's time chain, the forward scan,
 * the backward's reverse scan) have settings that the public calls always take at their
 * defaults.  Tests reach the other paths of those kernels through the calls below: each is
 * the public call of the same name with a leading `knobs` argument (NULL = the defaults).
 * The settings are arguments of the one call: the library keeps no state between calls.
 *
 *   lru_ticket_guess  fused RG-LRU kernel: each workgroup takes its tile from a ticket
 *                     counter and, while the atomic is in flight, loads the first operand
 *                     block of the tile it gets when tickets go in launch order, shifted by
 *                     this many tickets (default 0).  With a shift > 0 (nearly) every
 *                     workgroup guesses wrong and loads its own tile again; results must not
 *                     change.
 *   scan_direct_polls forward scan: polls of an unpublished predecessor summary before the
 *                     chunk computes that summary itself from memory (default 2048); < 0
 *                     ignores every published summary.  Results must not change.
 *   lookback_polls    fused RG-LRU kernel and reverse scan: polls of an unpublished
 *                     predecessor before the look-back gives up (default 2^20); < 0 gives up
 *                     at once.  Giving up writes NaN where the carry was needed and makes
 *                     rglru_workspace_status return RGLRU_ESTALL; every kernel still ends.
 *   lru_force_fused   bf16 RG-LRU layer of the forward: 1 runs the fused kernel whatever the
 *                     shape (default 0: the form the shape selects, which for shapes whose
 *                     fused tiles leave their last round of 256 CUs at most 60% full is the
 *                     gate projection then the scan).  Lets the tests reach the fused kernel
 *                     at every shape; the workspace sized for the shape's form suffices.
 */
#ifndef RGLRU_TESTING_H
#define RGLRU_TESTING_H

#include "../../include/rglru.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int lru_ticket_guess;
  int scan_direct_polls;
  int lookback_polls;
  int lru_force_fused;
} rglru_testing_knobs;

/* Fills *knobs with the settings every public call uses. */
void rglru_testing_default_knobs(rglru_testing_knobs* knobs);

int rglru_testing_fwd(const rglru_testing_knobs* knobs, int B, int T, int D, rglru_dtype io,
                      float c, const void* x, const void* conv_w, const float* conv_b,
                      const void* conv_state_in, const void* W_a, const void* W_x,
                      const float* b_a, const float* b_x, const float* lambda, const float* h0,
                      void* y, float* h_T, void* conv_state_out, void* ws, size_t ws_bytes,
                      hipStream_t stream);

int rglru_testing_scan(const rglru_testing_knobs* knobs, int B, int T, int D, rglru_dtype io,
                       const void* x, const void* conv_w, const float* conv_b,
                       const void* conv_state_in, const float* a, const float* beta,
                       const float* h0, void* y, float* h_T, void* ws, size_t ws_bytes,
                       hipStream_t stream);

int rglru_testing_bwd(const rglru_testing_knobs* knobs, int B, int T, int D, rglru_dtype io,
                      float c, const void* x, const void* conv_w, const float* conv_b,
                      const void* conv_state_in, const void* W_a, const void* W_x,
                      const float* b_a, const float* b_x, const float* lambda, const float* h0,
                      const void* dy, const float* dh_T, float* dx, float* dconv_w,
                      float* dconv_b, float* dW_a, float* dW_x, float* db_a, float* db_x,
                      float* dlambda, float* dh0, void* ws, size_t ws_bytes, hipStream_t stream);

int rglru_testing_block_fwd(const rglru_testing_knobs* knobs, int B, int T, int D, int R,
                            rglru_dtype io, float c, const void* x, const void* W_in,
                            const void* conv_w, const float* conv_b, const void* conv_state_in,
                            const void* W_a, const void* W_x, const float* b_a, const float* b_x,
                            const float* lambda, const float* h0, const void* W_out, void* out,
                            float* h_T, void* conv_state_out, void* ws, size_t ws_bytes,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RGLRU_TESTING_H */
