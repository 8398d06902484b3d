// Main loop of the bf16 MFMA GEMM shared by the gate projection, the fused RG-LRU kernel
// and the backward products: C_tile = A_tile B_tile^T with both operands K-contiguous.
//
// Tile: BM rows of A x BNR = 2 BC rows of B, WM x WN waves, each owning a
// (BM/WM) x (BNR/WN) block made of 32x32 v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulation).
// In gate mode the B tile holds BC rows of W_a followed by the same BC rows of W_x, and a
// wave's fragments pair them up, so z^a and z^x of one (row, channel) end in matching
// accumulator slots.  Operands stream through a STAGES-deep LDS ring filled by
// global_load_lds_dwordx4 (16 bytes per lane, no VGPR staging); an LDS row holds BK bf16 =
// CPR chunks of 16 bytes and chunk c of row r sits at chunk c ^ ((r / RP) % CPR) (RP rows
// per 256 bytes), so the 16-lane groups of every ds_read_b128 fragment fetch hit 16
// distinct 16-byte slots of the 64 banks.
#pragma once

#include "rglru_device.h"

namespace rglru {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Wait until at most N of this wave's vector-memory operations (the LDS DMA loads) are
// pending and all of its LDS operations are done, then meet the workgroup barrier.  A
// plain __syncthreads() would also drain every in-flight DMA stage (its fence waits for
// vmcnt(0)); the "memory" clobber keeps the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void wait_dma_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // The builtin wait (vmcnt(N) lgkmcnt(0), expcnt left at its maximum 7) is the one that
  // counts; it also tells the compiler's wait-count tracking what has completed (it cannot
  // see into asm), so later LDS reads get exact waits.  The asm adds the barrier, and its
  // memory clobber keeps memory accesses from moving across.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BM_, int BC_, int WM_, int WN_, bool PLAIN_, int BK_, int STAGES_>
struct GemmCfg {
  static constexpr int BM = BM_, BC = BC_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
  static constexpr bool PLAIN = PLAIN_;
  static constexpr int RB = BK * 2;                 // bytes per LDS row
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int RP = 256 / RB;               // rows per 256 bytes
  static constexpr int NW = WM * WN;
  static constexpr int BNR = 2 * BC;                // B-tile rows
  static constexpr int WTM = BM / WM, WTNR = BNR / WN;
  static constexpr int MF = WTM / 32, NF = WTNR / 32;
  static constexpr int ROWS = BM + BNR;
  static constexpr int STAGE = ROWS * RB;           // bytes per stage
  static constexpr int LDS_BYTES = STAGES * STAGE;
  static constexpr int RPI = 1024 / RB;             // rows per 1 KB DMA wave-instruction
  static constexpr int QPW = ROWS / RPI / NW;       // DMA instructions per wave per stage
  static constexpr int QA = BM / RPI / NW;          // ... of which load A rows
  static constexpr int QB1 = (BM + BC) / RPI / NW;  // gate mode: first W_x load
  static constexpr int KK = BK / 16;                // MFMA k-slices per k-step
  static_assert(WTM % 32 == 0 && WTNR % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((ROWS / RPI) % NW == 0 && (BM / RPI) % NW == 0 && ((BM + BC) / RPI) % NW == 0, "");
  static_assert(PLAIN || (BC / WN) % 32 == 0, "gate mode pairs 32-channel blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(STAGES >= 2 && (STAGES - 2) * QPW <= 63, "vmcnt range");
  static_assert(KK % 2 == 0, "k-slices per k-step must be even");
};

struct TileOperands {
  const bf16_t* A;      // rows a_row0 .. a_row0 + a_rows - 1 (clamped), row stride lda
  const bf16_t* A2;     // second A pass over the same K (dual mode) or NULL
  const bf16_t* B0;     // plain: B rows; gate: W_a rows
  const bf16_t* B1;     // gate: W_x rows
  int lda, ldb, K;
  int a_row0, a_rows;   // first global A row of the tile and valid rows (>= 1)
  int b_row0, b_rows;   // first global B row (gate: channel) and valid rows (>= 1)
};

// MFMAs LO .. HI-1 of a k-slice (fragment mf x fragment f, f fastest).
template <class C, int LO, int HI>
__device__ __forceinline__ void mfma_range(f32x16_t (&acc)[C::MF][C::NF], const bf16x8_t* af,
                                           const bf16x8_t* bfr) {
#pragma unroll
  for (int i = LO; i < HI; ++i) {
    const int mf = i / C::NF, f = i % C::NF;
    acc[mf][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mf], bfr[f], acc[mf][f], 0, 0, 0);
  }
}

// Scheduling groups for a region holding NM MFMAs and NR LDS reads: one MFMA, then reads
// and MFMAs alternating, then whatever is left of either.
template <int NM, int NR>
__device__ __forceinline__ void sched_reads_after_first_mfma() {
  constexpr int P = NR < NM - 1 ? NR : NM - 1;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  if constexpr (NR > P) __builtin_amdgcn_sched_group_barrier(0x100, NR - P, 0);
  if constexpr (NM - 1 > P) __builtin_amdgcn_sched_group_barrier(0x008, NM - 1 - P, 0);
}

// Scheduling groups for NM MFMAs with NR LDS reads spread in front of them.
template <int NM, int NR>
__device__ __forceinline__ void sched_reads_spread() {
  constexpr int Q = NR / NM, RM = NR % NM;
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, Q + 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
#pragma unroll
  for (int i = RM; i < NM; ++i) {
    if constexpr (Q > 0) __builtin_amdgcn_sched_group_barrier(0x100, Q, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// The operand DMA of one wave: per-lane source offsets (elements) of its global_load_lds
// instructions, and the issue of one k-step into its ring stage.
template <class C, bool DUAL>
struct GemmDma {
  uint32_t off[C::QPW];
  int KT1;   // k-steps per pass
  __device__ __forceinline__ GemmDma(const TileOperands& op, int lane, int wave) {
#pragma unroll
    for (int q = 0; q < C::QPW; ++q) {
      const int r = (q * C::NW + wave) * C::RPI + lane / C::CPR;
      const int pchunk = lane % C::CPR;
      if (q < C::QA) {
        const int gm = op.a_row0 + min(r, op.a_rows - 1);
        off[q] = uint32_t(gm) * uint32_t(op.lda) + uint32_t((pchunk ^ ((r / C::RP) % C::CPR)) * 8);
      } else {
        const int rb = r - C::BM;
        const int gn = op.b_row0 + min(C::PLAIN ? rb : rb % C::BC, op.b_rows - 1);
        off[q] = uint32_t(gn) * uint32_t(op.ldb) + uint32_t((pchunk ^ ((rb / C::RP) % C::CPR)) * 8);
      }
    }
    KT1 = op.K / C::BK;
  }
  __device__ __forceinline__ void issue(const TileOperands& op, unsigned char* lds, int wave,
                                        int kt) const {
    const bf16_t* abase = (DUAL && kt >= KT1) ? op.A2 : op.A;
    const int kofs = (DUAL && kt >= KT1 ? kt - KT1 : kt) * C::BK;
    unsigned char* sbase = lds + (kt % C::STAGES) * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::QPW; ++q) {
      const bf16_t* base = q < C::QA ? abase : ((!C::PLAIN && q >= C::QB1) ? op.B1 : op.B0);
      const bf16_t* gp = base + off[q] + kofs;
      __builtin_amdgcn_global_load_lds((void*)gp, (void*)(sbase + (q * C::NW + wave) * 1024), 16, 0, 0);
    }
  }
};

// Accumulate the tile into acc.  lds must hold C::LDS_BYTES; wave = wave index in the WG.
// first_issued: the caller has already issued k-step 0 (GemmDma::issue with the same op)
// and nothing else on the vector-memory counter since, apart from operations it waits for.
template <class C, bool DUAL>
__device__ __forceinline__ void gemm_mainloop(const TileOperands& op, unsigned char* lds, int lane,
                                              int wave, f32x16_t (&acc)[C::MF][C::NF],
                                              bool first_issued = false) {
  const int wm = wave / C::WN, wn = wave % C::WN;
  const GemmDma<C, DUAL> dma(op, lane, wave);
  const int KT = DUAL ? 2 * dma.KT1 : dma.KT1;
  auto issue = [&](int kt) { dma.issue(op, lds, wave, kt); };

  // LDS byte offsets of this lane's operand fragment rows
  int arow[C::MF], brow[C::NF];
#pragma unroll
  for (int mf = 0; mf < C::MF; ++mf) arow[mf] = (wm * C::WTM + mf * 32 + (lane & 31)) * C::RB;
#pragma unroll
  for (int f = 0; f < C::NF; ++f) {
    int base;
    if (C::PLAIN) {
      base = wn * C::WTNR + f * 32;
    } else {
      const int half = C::NF / 2;
      base = (f / half) * C::BC + wn * (C::BC / C::WN) + (f % half) * 32;
    }
    brow[f] = (C::BM + base + (lane & 31)) * C::RB;
  }
  const int swz = ((lane & 31) / C::RP) % C::CPR;
  const int khalf = lane >> 5;

#pragma unroll
  for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
    for (int f = 0; f < C::NF; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mf][f][v] = 0.f;

  auto load_frags = [&](int kt, int kk, bf16x8_t* af, bf16x8_t* bfr) {
    const unsigned char* sb = lds + (kt % C::STAGES) * C::STAGE;
    const int coff = ((kk * 2 + khalf) ^ swz) * 16;
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf) af[mf] = *reinterpret_cast<const bf16x8_t*>(sb + arow[mf] + coff);
#pragma unroll
    for (int f = 0; f < C::NF; ++f) bfr[f] = *reinterpret_cast<const bf16x8_t*>(sb + brow[f] + coff);
  };
  // Software pipeline: the fragments of the next k-slice are read from LDS while the MFMAs
  // of the current one run; the scheduling groups below pin the order (one MFMA first, then
  // reads and MFMAs alternating) so that the wait for a slice's fragments only covers reads
  // issued a whole slice earlier.  The barrier that hands over the next k-step sits in the
  // middle of the last slice's MFMAs, so the matrix core stays busy across it; after the
  // barrier every wave is done with k-step kt's buffer, which is refilled with k-step
  // kt + STAGES.  The final k-step is peeled off so that the loop body is the same on every
  // trip (a conditional tail inside the loop makes the compiler drain all LDS reads at the
  // loop header).
  constexpr int S = C::STAGES;
  constexpr int NM = C::MF * C::NF, NR = C::MF + C::NF, NM1 = NM / 2;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT && (s > 0 || !first_issued)) issue(s);
  if (S - 2 < KT) wait_dma_barrier<(S - 2) * C::QPW>();
  else wait_dma_barrier<0>();
  if (S - 1 < KT) issue(S - 1);
  bf16x8_t fa[2][C::MF], fb[2][C::NF];
  load_frags(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < KT - 1; ++kt) {
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const int cur = kk & 1;   // KK is even: slice 0 of every k-step lives in buffer 0
      if (kk + 1 < C::KK) {
        mfma_range<C, 0, NM>(acc, fa[cur], fb[cur]);
        load_frags(kt, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
        sched_reads_after_first_mfma<NM, NR>();
      } else {
        mfma_range<C, 0, NM1>(acc, fa[cur], fb[cur]);
        __builtin_amdgcn_sched_barrier(0);
        // k-step kt+1 has landed once at most min(S-2, KT-2-kt) newer k-steps pend
        if (kt + S - 1 < KT) wait_dma_barrier<(S - 2) * C::QPW>();
        else wait_dma_barrier<0>();
        if (kt + S < KT) issue(kt + S);
        __builtin_amdgcn_sched_barrier(0);
        mfma_range<C, NM1, NM>(acc, fa[cur], fb[cur]);
        load_frags(kt + 1, 0, fa[cur ^ 1], fb[cur ^ 1]);
        sched_reads_spread<NM - NM1, NR>();
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    const int cur = kk & 1;
    mfma_range<C, 0, NM>(acc, fa[cur], fb[cur]);
    if (kk + 1 < C::KK) {
      load_frags(KT - 1, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
      sched_reads_after_first_mfma<NM, NR>();
    }
  }
}

// Accumulator slot v of lane l holds tile row 8*(v/4) + 4*(l/32) + v%4 (within its 32-row
// block) and column l%32 (within its 32-column block).
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

}  // namespace rglru
