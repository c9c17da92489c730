// cce.hip -- Cut Cross-Entropy for MI355X (gfx950): kernels and the C ABI.
//
// What is computed follows "Cut Your Losses in Large-Vocabulary Language
// Models" (paper digest: "The Mathematical Decomposition", Algorithms 1-4,
// "Gradient Filtering"), the CCE blog post ("The decomposition", "Gradient
// filtering") and the kernel card "cut-cross-entropy" ("Method",
// "Correctness").  How it is computed is designed for CDNA4:
//
//   both      k_compact,   ignored rows moved behind the valid ones ("Cut Your
//             k_gather_rows Losses" digest, Table A1: ignored tokens dropped
//                          ahead of the loss); every kernel after them works
//                          on the compacted rows and skips tiles past them.
//   forward   k_fwd_lse    one workgroup per (256-token tile, vocabulary slab).
//                          256x256 bf16 MFMA logit tiles (fp32 accumulate,
//                          K = D brought into LDS by direct-to-LDS loads), every
//                          tile folded at once into a per-lane online (max,
//                          sum-exp) in registers; the lanes, then the waves,
//                          combine with shuffles / LDS and one (max, sum)
//                          partial per (slab, token) is written.  No logits
//                          leave the chip, no locks.
//             k_target     the target logit as an indexed dot, one wave per
//                          token.
//             k_fwd_merge  fixed-order merge of the slab partials -> lse, loss;
//                          fixed-order block sums for mean / sum.
//   backward  per vocabulary chunk (8192 or 16384 entries), one k_bwd_step
//             launch running four roles side by side, longest tiles first
//             (dE and dC of the previous chunk, then G-hat and the scaled
//             fp16 transpose of the C chunk for the next launch's dE):
//             G-hat        recompute the logit tile, G = exp(A - lse) - onehot,
//                          the wavefront-ballot filter per 32x32 unit, scale by
//                          the row's upstream gradient, round to fp16 and write
//                          the kept units of the chunk's G-hat in both
//                          orientations (for the next chunk's launch).
//             dC           dC[chunk] = G-hat^T E: every workgroup owns a
//                          disjoint 256-row vocabulary panel and reduces over
//                          all N tokens in registers, one bf16 write, no atomics.
//             dE           dE += G-hat C[chunk]: the chunks are the split-K
//                          slices of the vocabulary sum, accumulated in a fixed
//                          order into an fp32 buffer, cast to bf16 by the last.
//                          With very few dE tiles each chunk is also dealt over
//                          parts with their own buffers; k_de_final adds them.
//   sorting   k_vo_*       the average logit of every vocabulary entry and a
//                          bitonic sort by it ("Cut Your Losses" digest,
//                          "Vocabulary Sorting"); k_bwd_step<true> runs the
//                          backward with the vocabulary in a given order.
//   All three backward contractions are MFMA GEMMs whose K is the hidden
//   size, the tokens or the chunk; G-hat round-trips through a bounded
//   scratch rather than each tile read-modify-writing fp32 partials of dE and
//   dC over the full D.  Filtered units of G-hat are neither written nor read.
//
// Every reduction has a fixed order, so results are bitwise reproducible.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <type_traits>
#include <mutex>
#include <string>
#include <vector>

#include "cce.h"

namespace {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Workgroup tile of every contraction: BM rows (A operand) x BN columns
// (B operand); 8 waves, two per SIMD, each 128 rows x 64 columns: an 8 x 4
// grid of 16x16 output blocks of v_mfma_f32_16x16x32 (K = 32 per
// instruction), accumulators in 128 VGPRs.  Per flop the 16x16x32 form moves
// half the accumulator data of the 32x32x16 form; under the chip's power
// limit it sustains about 12% more throughput on random operands.  The K
// pipeline (depth of a step, LDS stages, refill policy) is a per-kernel
// choice: see Pipe below.  One workgroup per CU (128 KiB of LDS).
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int NWAVES = 8;                  // two per SIMD
constexpr int NTHREADS = 64 * NWAVES;
constexpr int WCOLS = BN / (NWAVES / 2);   // columns per wave: 2 row halves x NWAVES/2
constexpr int MB = 8;                      // 16-row MFMA blocks per wave (128 rows)
constexpr int NB = WCOLS / 16;             // 16-column MFMA blocks per wave
constexpr int RW = BM / NWAVES;            // operand rows each wave brings into LDS
// Wave w computes row half wave_m(w) (128 rows) and column quarter wave_n(w)
// (WCOLS columns).  The workgroup's waves are dealt to the 4 SIMDs round
// robin (w and w + 4 share one), so each SIMD gets one wave of each row half:
// where the MFMAs of filtered units are skipped, a wave's work depends on its
// row half only, and this gives every SIMD the same total.
__device__ __forceinline__ int wave_m(int w) { return (w >> 2) & 1; }
__device__ __forceinline__ int wave_n(int w) { return w & 3; }
constexpr int TR_STRIDE = BN + 8;       // C block in LDS for the transpose role (u16)
constexpr int UNIT = 32;                // filter unit: 32 tokens x 32 vocabulary entries
constexpr int CU = WCOLS / UNIT;        // column units per wave (2 MFMA blocks each)
// Backward vocabulary chunk: 16384 rows only while the G-hat scratch it
// implies (2 copies x N_pad x chunk fp16) stays within 256 MiB (N_pad <= 4096)
// and a launch has at least 128 dE workgroups (tiles x the parts each is
// dealt over), else 8192.  Larger chunks mean fewer launches (fewer tails)
// and fewer passes of the fp32 dE accumulator (measured: 8192 costs about 2%
// of the step at the Gemma-2-2B and GPT-OSS head shapes against 16384, and
// saves 328 / 608 MiB of workspace); a dE workgroup runs its whole part of
// the chunk as its K, so with few of them the launch cannot end before one
// of them does, and a shorter chunk shortens that pole.
constexpr int64_t VCHUNK_SMALL = 8192, VCHUNK_LARGE = 16384;
// Token blocks of the backward: past TB_MAX padded rows, blocks of at most
// TB_ROWS rows (the G-hat double buffer is then at most 2 x TB_ROWS x chunk).
constexpr int64_t TB_MAX = 16384, TB_ROWS = 8192;
__host__ __device__ constexpr int64_t vchunk_for(int64_t Npad, int64_t Dpad, int64_t parts) {
  return (Npad <= 4096 && (Npad / 256) * (Dpad / 256) * parts >= 128) ? VCHUNK_LARGE
                                                                        : VCHUNK_SMALL;
}
constexpr float LOG2E = 1.4426950408889634f;
constexpr int NCOUNT = 64;              // filter counters (spread over workgroups)
constexpr int OOB = 0x7ffffff0;         // buffer offset that always reads as zero

typedef __attribute__((address_space(3))) void *lds_ptr_t;

struct RowInfo {
  float lse2;    // lse * log2(e); +inf on rows whose G is not computed (exp2 gives 0)
  float gt;      // G at the target entry, p_t - 1 = expm1(t - lse) from the fp64 target logit
  int32_t tgt;   // target column, -1 if none
  int32_t live;  // 1 if the row's G is computed
};

__device__ __forceinline__ u16 f2bf(float f) {
  __bf16 b = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(u16, b);
}

__device__ __forceinline__ u16 f2h(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(u16, h);
}

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Power-of-two scale that maps a tensor whose largest |value| has the
// (fp32 / bf16) biased exponent eb into [2^13, 2^14): fp16 then holds every
// value with its full bf16 mantissa far from overflow.  Zero, inf and NaN
// give 1.
__device__ __forceinline__ float pow2_scale_e(int eb) {
  if (eb == 0 || eb == 255) return 1.0f;
  const int k = min(60, max(-60, 140 - eb));
  return __uint_as_float((uint32_t)(k + 127) << 23);
}
// 1 / pow2_scale_e(eb), exact (a power of two)
__device__ __forceinline__ float pow2_recip_e(int eb) {
  if (eb == 0 || eb == 255) return 1.0f;
  const int k = min(60, max(-60, 140 - eb));
  return __uint_as_float((uint32_t)(127 - k) << 23);
}
// ... of a bf16 maximum given by its magnitude bits
__device__ __forceinline__ float pow2_scale(uint32_t b) { return pow2_scale_e((int)((b >> 7) & 0xff)); }
__device__ __forceinline__ float pow2_recip(uint32_t b) { return pow2_recip_e((int)((b >> 7) & 0xff)); }
// ... of an fp32 maximum
__device__ __forceinline__ float pow2_scale_f(float m) {
  return pow2_scale_e((int)((__float_as_uint(m) >> 23) & 0xff));
}
__device__ __forceinline__ float pow2_recip_f(float m) {
  return pow2_recip_e((int)((__float_as_uint(m) >> 23) & 0xff));
}

// A per-call scalar written by an earlier launch (sigma, an amax): read
// through the constant address space at the start of a tile, so it is a
// scalar load that has long landed when the epilogue needs it.
__device__ __forceinline__ uint32_t ld_const_u32(const uint32_t *p) {
  typedef const __attribute__((address_space(4))) uint32_t *cp_t;
  return *(cp_t)(uintptr_t)p;
}

// G-hat is stored in fp16 as G * 2^15, before the row's upstream scale s_n:
// |G| <= 1 keeps it below 2^15 and every |G| above ~2e-9 stays a normal fp16
// number (11 significant bits instead of bf16's 8), whatever s_n is.  s_n
// enters dE as a per-row factor of the fp32 result and dC through its other
// operand, the power-of-two-scaled fp16 copy of s_n E_n; so no row's dE loses
// precision to the spread of the upstream gradients.
constexpr float GSCALE = 32768.0f;

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that consecutive logical tiles (which share operand panels) land on the
// same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int q = G >> 3, r = G & 7;
  const int xcd = bid & 7, local = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Logical tile L -> (a, b) on an A x B grid.  When A % 4 == 0 and B % 8 == 0
// tiles go in 4x8 blocks: the 32 workgroups an XCD runs at once share 4
// a-panels and 8 b-panels in its L2 instead of 1 and 32.
__device__ __forceinline__ void grouped(int L, int A, int B, int &a, int &b) {
  if ((A & 3) == 0 && (B & 7) == 0) {
    const int blk = L >> 5, w = L & 31, nb = B >> 3;
    a = ((blk / nb) << 2) + (w >> 3);
    b = ((blk % nb) << 3) + (w & 7);
  } else {
    a = L / B;
    b = L % B;
  }
}

// Logical tile L -> (a, b) for dC / dE, whose A panels (G-hat) are lighter
// than their B panels (the dense operand; only kept units of G-hat are
// loaded): strips of S b-panels (S = 4, 3 or 2, whichever divides B first,
// else 1), each walked a-major, so the 32 workgroups an XCD runs at once
// share about 32 / S a-panels and S b-panels (a third fewer distinct bytes
// past L2 than the 4 x 8 order at the kept fractions of the head shapes).
__device__ __forceinline__ void strips(int L, int A, int B, int &a, int &b) {
  const int S = (B & 3) == 0 ? 4 : (B % 3) == 0 ? 3 : (B & 1) == 0 ? 2 : 1;
  const int per = A * S, s = L / per, r = L - s * per;
  a = r / S;
  b = s * S + (r - a * S);
}

// The compacted row count, written by an earlier launch and read by every
// workgroup before its tile starts: a scalar load through the constant
// address space (the scalar cache starts each launch invalidated), so no
// vector-memory wait sits in front of the tile's first loads.
__device__ __forceinline__ int load_nvalid(const int64_t *p) {
  typedef const __attribute__((address_space(4))) int64_t *cp_t;
  return (int)*(cp_t)(uintptr_t)p;
}

// Token tiles that hold compacted (valid) rows, rounded up to a multiple of
// `group` (the launch order's tile groups) and capped at the launch's count.
// A launch sized for all rows numbers only these tiles: the hardware deals
// consecutive workgroup ids to the XCDs in turn, so the ids past them (which
// exit at once) are spread over every XCD and so is the work.
__device__ __forceinline__ int live_tiles(int nvalid, int tiles, int group) {
  const int t = (nvalid + 255) / 256;
  return min(tiles, (t + group - 1) / group * group);
}

// Buffer resource for a tile: base and size are workgroup-uniform; the
// readfirstlanes put them in scalar registers even where the compiler's
// uniformity analysis loses track (a divergent descriptor would wrap every
// load in a waterfall loop).  bytes is < 2^31 for every tile (host-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int nb = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, nb,
                                           0x00020000);
}

// ---------------------------------------------------------------------------
// GEMM core: acc[256 x 256] = A[256 x K] . B[256 x K]^T, both K-contiguous
// (row-major, row stride ld bytes).
//
// Each K-step of BK is brought straight from global memory into LDS by
// buffer_load_dwordx4 ... lds (lane i of an instruction fills bytes
// 16i..16i+15 of a 1 KiB LDS block): no staging registers.  Rows past the
// tile's valid rows read zero (buffer range check); with ktail, 8-element
// chunks at k >= K read zero too.
//
// Fragments are read one K-step ahead: step kt multiplies the fragments of
// stage kt (already in registers) while reading those of stage kt + 1, each
// fragment register refilled right after the last MFMA that reads it.  One
// barrier per step makes stage kt + 1 visible and frees a buffer for the
// loads of a later stage: the step's own buffer after a full LDS wait
// (LAG 0), or the previous step's, whose reads every wave has consumed
// (LAG 1: LDS reads stay in flight across the barrier).  With UNROLL the
// step loop is unrolled NSTAGE times so each stage's LDS offset is a
// constant; the in-stage offsets being masked to the stage, the compiler
// can tell one stage's loads from another stage's reads and deal the loads
// out between the MFMAs.
//
// LDS has 64 four-byte banks.  A 16-lane group of ds_read_b128 reads 16
// consecutive tile rows at one chunk index; storing chunk c of row r at
// slot c ^ ((r / RPL) & (CHR - 1)) puts the 16 rows on 16 distinct 16-byte
// bank groups.
// ---------------------------------------------------------------------------
template <int BK_, int NSTAGE_, int LAG_, bool UNROLL_>
struct Pipe {
  static constexpr int BK = BK_;          // K-step depth: 32 or 64
  static constexpr int NSTAGE = NSTAGE_;  // LDS stage buffers
  static constexpr int LAG = LAG_;        // refill the buffer of step kt - LAG
  static constexpr bool UNROLL = UNROLL_;
  static constexpr int CHR = BK / 8;      // 16-byte chunks per tile row
  static constexpr int RPB = 64 / CHR;    // tile rows per 1 KiB direct-to-LDS block
  static constexpr int RPL = 128 / BK;    // tile rows per 256-byte LDS bank row
  static constexpr int STAGE = (BM + BN) * BK;  // u16 elements per stage
  static constexpr int LDS = NSTAGE * STAGE;
  static constexpr int LPS = 2 * (RW / RPB);    // direct-to-LDS loads per thread per stage
  static constexpr int PRO = NSTAGE - LAG;      // stages loaded before the loop
  static constexpr int KS = BK / 32;            // MFMA sub-steps per step
  static_assert(LAG == 0 || NSTAGE >= 3, "refilling the previous buffer needs 3 stages");
  static_assert((STAGE & (STAGE - 1)) == 0, "stage size must be a power of two");
  static_assert(!UNROLL || LAG == 1 || NSTAGE == 2, "unrolled loop policy");
  // without UNROLL every barrier waits for all loads (NSTAGE - LAG == 2)
  static_assert(UNROLL || NSTAGE - LAG == 2, "rolled loop policy");
};
// Forward logits: 32-deep steps, four stages, loads spread over each step.
// PipeB: the 64-deep step geometry (swizzle, loads per stage) of the
// backward's loop (mainloop_sp), which lays out its buffers itself.
using PipeF = Pipe<32, 4, 1, true>;
using PipeB = Pipe<64, 2, 0, false>;
// The backward's loop (G-hat recompute, dC, dE): 64-deep steps, three A and
// two B buffers of 32 KiB, the whole 160 KiB of LDS.
constexpr int B3_ASZ = BM * 64, B3_BSZ = BN * 64;  // u16 per buffer
constexpr int B3_LDS = 3 * B3_ASZ + 2 * B3_BSZ;
constexpr int LDS_MAIN = PipeF::LDS > B3_LDS ? PipeF::LDS : B3_LDS;

template <class P>
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row / P::RPL) & (P::CHR - 1));
}

// Wave w brings rows [RW*w, RW*w + RW) of a 256-row operand tile (op 0: A,
// 1: B) into stage buffer `stage` for the K-step starting at k0; chunks at
// k >= K read as zero without a memory request.
template <class P>
__device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t rs, int ld_bytes, int k0, int K,
                                           u16 *lds, int stage, int op, int w, int l) {
#pragma unroll
  for (int j = 0; j < RW / P::RPB; ++j) {
    const int r = RW * w + P::RPB * j + l / P::CHR;
    const int c = (l & (P::CHR - 1)) ^ ((r / P::RPL) & (P::CHR - 1));
    const int kk = k0 + c * 8;
    const int off = r * ld_bytes + kk * 2;
    const int use = kk < K ? off : OOB;
    u16 *dst = lds + stage * P::STAGE +
               ((op * BM * P::BK + (RW * w + P::RPB * j) * P::BK) & (P::STAGE - 1));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, use, 0, 0, 0);
  }
}

template <class P>
__device__ __forceinline__ u32x4 lfrag(const u16 *lds, int stage, int op, int row, int chunk) {
  return *reinterpret_cast<const u32x4 *>(
      lds + stage * P::STAGE +
      ((op * BM * P::BK + row * P::BK + swz<P>(row, chunk) * 8) & (P::STAGE - 1)));
}

// One 16x16x32 MFMA.  Operand lane layout: lane l holds row (A) / column (B)
// l & 15 at the 8 consecutive k of chunk l >> 4; the result puts rows
// 4 * (l >> 4) .. + 3 of column l & 15 in lane l.
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// lgkmcnt in bits 11:8), all with lgkmcnt(0).
__host__ __device__ constexpr int wait_vm(int n) {
  return (n & 15) | ((n >> 4) << 14) | 0x0070;  // vmcnt(n) expcnt(7) lgkmcnt(0)
}
constexpr int WAIT_VM0 = wait_vm(0);

// Workgroup barrier for the K-loop.  __syncthreads() carries a release fence
// that waits for every outstanding global load -- including the stages that
// are meant to stay in flight -- so the loop uses a bare s_barrier after
// its own s_waitcnt; the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Filter flags of a G-hat operand (mainloop_sp): fw + g * fstride points at
// the 8-byte words of the 4-row-unit group g of the tile (g = 0, 1 for rows
// 0-127, 128-255); word j covers the k range [64j, 64j + 64) and its byte
// ku*4 + u is 1 if the 32x32 unit (row unit u of the group, k unit 2j + ku)
// is kept.  Chunks of filtered units are never loaded (they arrive as zeros),
// so those units cost neither memory traffic nor reads of stale G-hat, and
// their MFMAs are skipped: a wave's 128 rows are one group, so the word of a
// step says for each of its 4 row units and 2 k units whether its 2 x NB
// MFMAs run (a wave-uniform scalar branch; skipped products are exact zeros).
// Rows of a tile in groups of 4 row units (128 rows): the group holding wave
// w's loaded rows, and the position of its first row unit in the group.
constexpr int LOAD_UNITS = (RW + 31) / 32;  // row units a wave loads: 2 or 1
__device__ __forceinline__ int load_group(int w) { return (RW * w) / 128; }

// Chunk-major loads of G-hat (mainloop_sp, ALK): wave w brings k unit w >> 2
// of row units 2 (w & 3), + 1 (mod 4) of the 128-row half (w & 3) / 2; bit
// b of the result is row unit 2 (w & 3) + b.
__device__ __forceinline__ uint32_t keep_bits_cm(uint64_t word, int w) {
  const int u0 = (2 * (w & 3)) & 3;
  const uint32_t h = (uint32_t)(word >> (32 * (w >> 2)));
  return ((h >> (8 * u0)) & 1u) | (((h >> (8 * u0 + 8)) & 1u) << 1);
}

__device__ __forceinline__ uint32_t keep_bits(uint64_t word, int w) {
  const int u0 = ((RW * w) / 32) & 3;  // first of the wave's row units in its group
  const int sh = u0 * 8;
  const uint32_t lo = (uint32_t)word, hi = (uint32_t)(word >> 32);
  uint32_t k0 = (lo >> sh) & 1u, k1 = (hi >> sh) & 1u;  // k units 2j, 2j + 1
  if (LOAD_UNITS > 1) {
    k0 |= ((lo >> (sh + 8)) & 1u) << 1;
    k1 |= ((hi >> (sh + 8)) & 1u) << 1;
  } else {
    k0 |= k0 << 1;  // one row unit: both row-bit positions mean it
    k1 |= k1 << 1;
  }
  return k0 | (k1 << 2);
}

// Scheduling of a step with one sub-step (32-deep), in two halves so that no
// refill is read right before its use: first the left column blocks
// (nb < NB / 2) of every row block, two MFMAs per slot, then their B
// refills; then the right column blocks, each row block's two MFMAs followed
// by its A refill; the right B refills last (used in the next step's second
// half).  Loads as in sched_step, over S = 2 * MB slots.
template <int I, int NV, int SP>
__device__ __forceinline__ void sched_halves() {
  constexpr int S = 2 * MB;
  if constexpr (I < S) {
    constexpr int nv = I < SP ? (((I + 1) * NV + SP - 1) / SP - (I * NV + SP - 1) / SP) : 0;
    __builtin_amdgcn_sched_group_barrier(0x008, NB / 2, 0);  // MFMAs
    if constexpr (I >= MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // A refill
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);  // loads
    if constexpr (I % MB == MB - 1)
      __builtin_amdgcn_sched_group_barrier(0x100, NB / 2, 0);  // B refills
    sched_halves<I + 1, NV, SP>();
  }
}

// The prologue's loads of a tile without filter flags, issued ahead of time:
// a caller with several tiles per workgroup sends the next tile's first
// stages before it runs the current tile's epilogue, then calls mainloop
// with PRO_DONE.  The caller's own loads in between must not be global
// reads (the wait at the top of the loop counts only these).
template <class P>
__device__ __forceinline__ void mainloop_prologue(__amdgpu_buffer_rsrc_t rsA, int lda_bytes,
                                                  __amdgpu_buffer_rsrc_t rsB, int ldb_bytes,
                                                  int K, u16 *lds) {
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int KT = (K + P::BK - 1) / P::BK;
  __syncthreads();  // the previous user of the stages is done with them
#pragma unroll
  for (int s = 0; s < P::PRO; ++s) {
    issue_rows<P>(rsA, lda_bytes, s * P::BK, s < KT ? K : 0, lds, s, 0, w, l);
    issue_rows<P>(rsB, ldb_bytes, s * P::BK, s < KT ? K : 0, lds, s, 1, w, l);
  }
}

// The forward logit tiles and the G-hat recompute: an unrolled pipeline of
// NSTAGE stages refilling the buffer of step kt - LAG, no filter flags.
template <class P, bool F16, bool PRO_DONE = false>
__device__ __forceinline__ void mainloop(__amdgpu_buffer_rsrc_t rsA, int lda_bytes,
                                         __amdgpu_buffer_rsrc_t rsB, int ldb_bytes, int K,
                                         u16 *lds, f32x4 (&acc)[MB][NB]) {
  static_assert(P::UNROLL && P::KS == 1, "one 32-deep sub-step per unrolled step");
  constexpr int BK = P::BK, NSTAGE = P::NSTAGE, LAG = P::LAG;
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave_m(w), wn = wave_n(w);

  const int KT = (K + BK - 1) / BK;
  if (!PRO_DONE) __syncthreads();  // the previous user of the stages is done with them
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (KT == 0) return;
  constexpr int NV = P::LPS;  // loads per stage and thread
  // the loads of stage kt + 1 went out NSTAGE - LAG - 1 steps before step kt
  constexpr int WAIT_STEADY =
      LAG ? (wait_vm(NV * (NSTAGE - LAG - 2)) | 0x0f00) : wait_vm(NV * (NSTAGE - 2));
  // Prologue: every buffer but (LAG) the last is filled.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!PRO_DONE) {
#pragma unroll
    for (int s = 0; s < P::PRO; ++s) {
      issue_rows<P>(rsA, lda_bytes, s * BK, s < KT ? K : 0, lds, s, 0, w, l);
      issue_rows<P>(rsB, ldb_bytes, s * BK, s < KT ? K : 0, lds, s, 1, w, l);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(NV * (P::PRO - 1)));  // stage 0 landed
  stage_barrier();

  const int arow = wm * 128 + (l & 15);
  const int brow = wn * WCOLS + (l & 15);
  const int kq = l >> 4;  // the lane's 8-element chunk of the 32-deep step
  // stage 0's fragments, read in the order the loop refills them (so the
  // waits at the loop head count outstanding reads alike on both paths in)
  u32x4 fa[MB], fb[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    fa[mb] = lfrag<P>(lds, 0, 0, arow + mb * 16, kq);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    fb[nb] = lfrag<P>(lds, 0, 1, brow + nb * 16, kq);
    __builtin_amdgcn_sched_barrier(0);
  }
  // One step; b = kt % NSTAGE (a constant: the loop is unrolled NSTAGE times).
  auto step = [&](int kt, int b) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(WAIT_STEADY);
    stage_barrier();
    {
      const int kn = kt + NSTAGE - LAG;
      const int rb = (b + NSTAGE - LAG) % NSTAGE;
      issue_rows<P>(rsA, lda_bytes, kn * BK, kn < KT ? K : 0, lds, rb, 0, w, l);
      issue_rows<P>(rsB, ldb_bytes, kn * BK, kn < KT ? K : 0, lds, rb, 1, w, l);
    }
    const int nbuf = (b + 1) % NSTAGE;
    // two column halves: the left half's B refills are read mid-step, not
    // right before the next step's first MFMA (sched_halves)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = h * NB / 2; nb < (h + 1) * NB / 2; ++nb)
          acc[mb][nb] = mfma16<F16>(fa[mb], fb[nb], acc[mb][nb]);
        if (h == 1) fa[mb] = lfrag<P>(lds, nbuf, 0, arow + mb * 16, kq);
      }
#pragma unroll
      for (int nb = h * NB / 2; nb < (h + 1) * NB / 2; ++nb)
        fb[nb] = lfrag<P>(lds, nbuf, 1, brow + nb * 16, kq);
    }
    // A refilled buffer is read NSTAGE - LAG - 1 steps later: the loads are
    // spread over the whole step when that leaves a step or more of slack,
    // over its first half with less.
    constexpr int SP = NSTAGE - LAG >= 3 ? 2 * MB : MB;
    sched_halves<0, NV, SP>();
  };
  // steps past KT (up to the next multiple of NSTAGE) multiply stages that
  // were loaded as zeros.  One copy of the unrolled body: peeling the first
  // steps (to start from a zero accumulator input) doubled the code the
  // register allocator has to fit around the epilogue's state.
  for (int k0 = 0; k0 < KT; k0 += NSTAGE) {
#pragma unroll
    for (int b = 0; b < NSTAGE; ++b) step(k0 + b, b);
  }
  // drain the loads of the zero-filled stages past the end before the LDS is
  // handed to an epilogue
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
}

// The backward's contractions on 64-deep steps with three A and two B
// buffers of 32 KiB (B(s + 2) and A(s + 3) issued at step s): the G-hat
// recompute (FLAGS false: A = a chunk of C, B = E, both row-major bf16) and
// dC / dE (FLAGS: A = G-hat in 8-wide k blocks (ABLK) with filter flags,
// filtered units neither loaded nor multiplied; B = the dense scaled-fp16
// operand).  Laid out so that the MFMA pipe does not wait for the step's
// bookkeeping:
//  * each step starts with the MFMAs of its first unit, issued before the
//    barrier (they read registers only), so the barrier wait overlaps them;
//  * the loads go out one at a time between units' MFMAs (a burst of loads
//    fills the address queue and stalls the wave while its MFMAs wait behind
//    them), each offset a per-lane constant plus a per-step scalar;
//  * with FLAGS the refill reads of a unit's A fragments go out right after
//    its MFMAs and only where the next step keeps that unit (the step head
//    waits for every read anyway, so skipped reads cost nothing and save LDS
//    time), and a tile whose every step is active runs a loop without the
//    search for the next active step.
// Layouts of the A operand (AL): row-major rows of lda_bytes (ALR); G-hat in
// 8-wide blocks along K (ALK: element (r, k) at ((k / 8) * rows + r) * 8 +
// k % 8, `ablk` the tile's first row in block column 0, lda_bytes the
// distance between block columns); or G-hat in 8-wide blocks along the tile's
// rows (ALT: element (r, k) at ((r / 8) * rows + k) * 8 + r % 8 -- the copy
// dE reads, taken by dC with its rows and K swapped: `ablk` the first of the
// tile's 32 row blocks at k = 0, lda_bytes the distance between row blocks).
// ALT is brought in one row block x 64 k (1 KiB, contiguous) per load and
// read with transposing LDS reads (ds_read_b64_tr_b16): each gives a lane 4
// consecutive k of one row, two of them an MFMA operand's 8.
constexpr int ALR = 0, ALK = 1, ALT = 2;

template <bool FLAGS, bool F16, int AL, bool BBLK = false, bool GATHER = false>
__device__ __forceinline__ bool mainloop_sp(__amdgpu_buffer_rsrc_t rsA, int lda_bytes,
                                            __amdgpu_buffer_rsrc_t rsB, int ldb_bytes, int K,
                                            u16 *lds, f32x4 (&acc)[MB][NB],
                                            const uint64_t *__restrict__ fw = nullptr,
                                            int fstride = 0, const u16 *ablk = nullptr,
                                            bool scan = false, const u16 *bblk = nullptr,
                                            const int32_t *__restrict__ gidx = nullptr,
                                            int grows = 0, int gV = 0) {
  using P = PipeB;
  constexpr int BK = P::BK, KS = P::KS;
  constexpr int NL = RW / P::RPB;  // direct-to-LDS loads per thread per operand per stage
  static_assert(NL == MB / 2, "one A load per row unit of the second sub-step");
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave_m(w), wn = wave_n(w);
  const int KT = (K + BK - 1) / BK;
  u16 *const bbase = lds + 3 * B3_ASZ;
  __syncthreads();  // the previous user of the LDS is done with it
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (KT == 0) return false;

  typedef const __attribute__((address_space(4))) uint64_t *cword_t;
  // the keep word of the rows this wave loads (ALK: quarter w & 3 of the
  // tile, in row half (w & 3) / 2) and the MFMA word of its row half
  const int lgrp = AL == ALK ? (w & 3) >> 1 : load_group(w);
  const cword_t fwl = (cword_t)(uintptr_t)(fw + (FLAGS ? (int64_t)lgrp * fstride : 0));
  const cword_t fwc = (cword_t)(uintptr_t)(fw + (FLAGS ? (int64_t)wm * fstride : 0));
  const int wlast = KT - 1;
  // without FLAGS every unit is kept: the words read as all ones
  auto wl = [&](int s) __attribute__((always_inline)) { return FLAGS ? fwl[min(s, wlast)] : ~0ull; };
  auto wc = [&](int s) __attribute__((always_inline)) { return FLAGS ? fwc[min(s, wlast)] : ~0ull; };

  // Per-lane parts of the load offsets.  Row-major operands (ALR, and B
  // without BBLK): load j of a thread fills tile row r_j = RW*w + RPB*j +
  // l/CHR at 16-byte chunk c_j (XOR-swizzled); in a step that chunk holds
  // k = 8 c_j .. 8 c_j + 7 of the step.  Operands stored in 8-wide k blocks
  // (ALK, BBLK) come in chunk-major: load j of wave w brings the 64 rows of
  // quarter w & 3 at chunk 4 (w >> 2) + j, 1 KiB contiguous in memory and in
  // LDS (element (r, chunk c) of a buffer at (c * 256 + r) * 16 bytes; the
  // 16 rows a ds_read_b128 group reads are 256 contiguous bytes, so no
  // swizzle is needed).  Those loads take one k unit of two row units: lane
  // l's row unit is bit l >> 5 of the keep bits (keep_bits_cm).
  int aoff[NL], boff[NL], kofs[NL], bkofs[NL];
  uint32_t kbit[NL];
  const int rq = 64 * (w & 3) + l;  // chunk-major: the lane's row
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int r = RW * w + P::RPB * j + l / P::CHR;
    const int c = (l & (P::CHR - 1)) ^ ((r / P::RPL) & (P::CHR - 1));
    const int cq = 4 * (w >> 2) + j;  // chunk-major: the load's chunk
    // ALK: within the step's 8 block columns of A; ALR: plus the step's k0 * 2
    aoff[j] = AL == ALK ? rq * 16 + cq * lda_bytes : r * lda_bytes + c * 16;
    kofs[j] = AL == ALK ? cq * 8 : c * 8;
    kbit[j] = AL == ALK ? 1u << (l >> 5) : 1u << ((((c * 8) >> 5) & 1) << 1 | ((r >> 5) & 1));
    if constexpr (GATHER) {
      // row r of the A tile is row gidx[r] of rsA; rows r >= grows and
      // indices outside [0, gV) read as zeros (offset -1)
      const int g = r < grows ? gidx[r] : -1;
      aoff[j] = (g >= 0 && g < gV) ? g * lda_bytes + c * 16 : -1;
    }
    // BBLK: within the step's 8 block columns of B; else plus the step's k0 * 2
    boff[j] = BBLK ? rq * 16 + cq * ldb_bytes : r * ldb_bytes + c * 16;
    bkofs[j] = BBLK ? cq * 8 : c * 8;
    if constexpr (AL == ALT) {
      // load j brings row block 4w + j (the wave's row unit) at the step's 64
      // k; lane l takes k = l ^ (4 (block & 1)) (a swizzle that keeps the
      // transposing reads conflict-free), landing at LDS slot l of the block
      const int vb = 4 * w + j, kl = l ^ (4 * (vb & 1));
      aoff[j] = vb * lda_bytes + kl * 16;
      kofs[j] = kl;
      kbit[j] = 1u << ((kl >> 5) << 1);
    }
  }
  // this wave's first load in an A / B buffer (then + ldst_j * j)
  u16 *const adst = AL == ALK ? lds + (4 * (w >> 2) * BM + 64 * (w & 3)) * 8 : lds + RW * w * BK;
  u16 *const bdst = BBLK ? bbase + (4 * (w >> 2) * BN + 64 * (w & 3)) * 8 : bbase + RW * w * BK;
  constexpr int ASTEP = AL == ALK ? BM * 8 : P::RPB * BK;  // u16 between a wave's loads
  constexpr int BSTEP = BBLK ? BN * 8 : P::RPB * BK;
  // load j of A(s) into A buffer ab, chunks of filtered units (keep bits kb)
  // read as zero; rs is the step's descriptor (arsrc)
  auto arsrc = [&](int s) __attribute__((always_inline)) {
    if constexpr (AL == ALK)
      return make_rsrc(ablk + (int64_t)s * (BK / 8) * (lda_bytes / 2), (int64_t)(BK / 8) * lda_bytes);
    else if constexpr (AL == ALT)
      return make_rsrc(ablk + (int64_t)s * BK * 8, (int64_t)(BM / 8) * lda_bytes);
    else
      return rsA;
  };
  auto issueA1 = [&](__amdgpu_buffer_rsrc_t rs, int s, int ab, uint32_t kb, int j)
      __attribute__((always_inline)) {
    const int Ks = s < KT ? K - s * BK : 0;  // k within the step below this are real
    const int off = AL == ALR ? aoff[j] + s * BK * 2 : aoff[j];
    const int use =
        (kofs[j] < Ks && (!FLAGS || (kb & kbit[j])) && (!GATHER || aoff[j] >= 0)) ? off : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_ptr_t)(adst + ab * B3_ASZ + ASTEP * j), 16, use, 0, 0, 0);
  };
  auto kbits = [&](uint64_t word) __attribute__((always_inline)) {
    return AL == ALK ? keep_bits_cm(word, w) : keep_bits(word, w);
  };
  auto issueA = [&](int s, int ab, uint32_t kb) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = arsrc(s);
#pragma unroll
    for (int j = 0; j < NL; ++j) issueA1(rs, s, ab, kb, j);
  };
  // BBLK: the step's 8 block columns of B (per-step descriptor, so the
  // offsets stay small whatever K is)
  auto brsrc = [&](int s) __attribute__((always_inline)) {
    if constexpr (BBLK)
      return make_rsrc(bblk + (int64_t)s * (BK / 8) * (ldb_bytes / 2), (int64_t)(BK / 8) * ldb_bytes);
    else
      return rsB;
  };
  auto issueB1 = [&](int s, int bb, int j) __attribute__((always_inline)) {
    const int Ks = s < KT ? K - s * BK : 0;
    const int use = bkofs[j] < Ks ? (BBLK ? boff[j] : boff[j] + s * BK * 2) : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        brsrc(s), (lds_ptr_t)(bdst + bb * B3_BSZ + BSTEP * j), 16, use, 0, 0, 0);
  };
  auto issueB = [&](int s, int bb) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NL; ++j) issueB1(s, bb, j);
  };
  const int arow = wm * 128 + (l & 15);
  const int brow = wn * WCOLS + (l & 15);
  const int kq = l >> 4;
  auto frag = [&](const u16 *buf, int row, int chunk) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4 *>(buf + row * BK + swz<P>(row, chunk) * 8);
  };
  // ALT: the A fragment of MFMA row block mb, sub-step kk.  Within each
  // 16-lane group, output lane i's element e comes from element i & 3 of the
  // 8 bytes lane 4e + (i >> 2) addresses, so lane 4e + q points at k = kbase
  // + e, rows 4q .. 4q + 3 of the 16: lane i then holds row i at k = kbase ..
  // kbase + 3.  Row block vb = 2 mb + (q >> 1) (+ the wave's row half), slot
  // k ^ (4 (vb & 1)); kbase = 32 kk + 8 (l >> 4), then + 4.
  const int tq = (l & 15) & 3, te = (l & 15) >> 2, tg = l >> 4;
  const int tbase = ((wm * 16 + (tq >> 1)) * 64 + 8 * tg + te) * 8 + 4 * (tq & 1);
  const int tsw = 4 * (tq >> 1);  // the swizzle of the lane's row block
  auto fragT = [&](const u16 *buf, int mb, int kk) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_t;
    const u16 *p = buf + tbase + mb * 2 * 64 * 8 + kk * 32 * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p + tsw * 8));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p + (4 - tsw) * 8));
    u32x4 o;
    o.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    o.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    o.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    o.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return o;
  };
  // chunk-major buffers (ALK, BBLK): 16 rows at one chunk, 256 contiguous bytes
  auto fragC = [&](const u16 *buf, int row, int chunk) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4 *>(buf + (chunk * BM + row) * 8);
  };
  auto afrag = [&](const u16 *buf, int mb, int kk) __attribute__((always_inline)) {
    if constexpr (AL == ALT) return fragT(buf, mb, kk);
    else if constexpr (AL == ALK) return fragC(buf, arow + mb * 16, kk * 4 + kq);
    else return frag(buf, arow + mb * 16, kk * 4 + kq);
  };
  auto bfrag = [&](const u16 *buf, int nb, int kk) __attribute__((always_inline)) {
    if constexpr (BBLK) return fragC(buf, brow + nb * 16, kk * 4 + kq);
    else return frag(buf, brow + nb * 16, kk * 4 + kq);
  };

  // K-steps where neither row half of the tile keeps a unit would load A as
  // zeros, skip every MFMA and still pay a barrier and the B loads; the loop
  // walks only the active steps.  Bit s of act: step s holds a kept unit,
  // taken from the two row halves' MFMA words by one vector load per lane
  // and a ballot per 64 steps.  Past 64 * AW steps (or without flags) every
  // step is walked, and so it is when the caller knows every unit is kept
  // (scan false: the contraction is unfiltered); a tile whose every step is
  // active (the common case under a peaked softmax) walks them all without
  // the per-step search.
  constexpr int AW = 4;
  uint64_t act[AW];
  bool walk_all = !FLAGS || !scan || KT > 64 * AW;
  bool any = true;  // some step is walked
  if (!walk_all) {
    bool full = true;
#pragma unroll
    for (int q = 0; q < AW; ++q) {
      const int s = q * 64 + l;
      uint64_t x = 0ull;
      if (s < KT) x = fw[s] | fw[fstride + s];
      act[q] = __ballot(x != 0ull);
      const int n = min(64, max(0, KT - q * 64));
      const uint64_t need = n == 64 ? ~0ull : ((1ull << n) - 1ull);
      full = full && (act[q] & need) == need;
    }
    walk_all = full;
    any = (act[0] | act[1] | act[2] | act[3]) != 0ull;
  }
  auto next_active = [&](int s) __attribute__((always_inline)) {
    if (s >= KT) return s;
    const int qs = s >> 6;
    const uint64_t ws = qs == 0 ? act[0] : qs == 1 ? act[1] : qs == 2 ? act[2] : act[3];
    if ((ws >> (s & 63)) & 1ull) return s;
    int r = KT;
#pragma unroll
    for (int q = AW - 1; q >= 0; --q) {
      uint64_t m = act[q];
      if (s >= (q + 1) * 64) m = 0ull;
      else if (s > q * 64) m &= ~0ull << (s - q * 64);
      if (m) r = q * 64 + (int)__builtin_ctzll(m);
    }
    return r;
  };

  // the MFMAs of row unit u (2 row blocks) for sub-step kk
  auto unit_mfma = [&](int kk, int u, const u32x4 (&fa)[KS][MB], const u32x4 (&fb)[KS][NB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[2 * u + a][nb] = mfma16<F16>(fa[kk][2 * u + a], fb[kk][nb], acc[2 * u + a][nb]);
  };

  auto run = [&](auto all_tag) __attribute__((always_inline)) {
    constexpr bool ALL = decltype(all_tag)::value;
    auto nxt = [&](int s) __attribute__((always_inline)) {
      if constexpr (ALL) return s;
      else return next_active(s);
    };
    int s0 = nxt(0);
    int s1 = nxt(s0 + 1);
    int s2 = nxt(s1 + 1);
    int s3 = nxt(s2 + 1);
    // prologue: A(s0) B(s0) A(s1) B(s1) A(s2); keep words of s0..s2, MFMA
    // words of s0, s1; in flight into the loop the keep word of s3 and the
    // MFMA word of s2
    const uint64_t kw0 = wl(s0), kw1 = wl(s1), kw2 = wl(s2);
    uint64_t fc = wc(s0), fcn = wc(s1);
    uint64_t kwf = wl(s3), fcf = wc(s2);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    issueA(s0, 0, kbits(kw0));
    issueB(s0, 0);
    issueA(s1, 1, kbits(kw1));
    issueB(s1, 1);
    issueA(s2, 2, kbits(kw2));
    __builtin_amdgcn_s_waitcnt(wait_vm(3 * NL));  // A(s0), B(s0) landed
    stage_barrier();
    u32x4 fa[KS][MB], fb[KS][NB];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) fa[kk][mb] = afrag(lds, mb, kk);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) fb[kk][nb] = bfrag(bbase, nb, kk);
    }
    int ab = 0, bb = 0;  // buffers of the step in registers (A: 3 in turn, B: 2)
    while (s0 < KT) {
      const int an = ab == 2 ? 0 : ab + 1, bn = bb ^ 1;  // buffers of step s1
      const u16 *ar = lds + an * B3_ASZ, *br = bbase + bn * B3_BSZ;
      auto kept = [&](uint64_t word, int kk, int u) __attribute__((always_inline)) {
        return !FLAGS || ((uint32_t)(word >> (kk * 32 + u * 8)) & 1u) != 0u;
      };
      // refill unit u's A fragments of sub-step kk from stage s1 where the
      // next step keeps it
      auto refill_unit = [&](int kk, int u) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        if (kept(fcn, kk, u)) {
          fa[kk][2 * u] = afrag(ar, 2 * u, kk);
          fa[kk][2 * u + 1] = afrag(ar, 2 * u + 1, kk);
        }
        __builtin_amdgcn_s_setprio(0);
      };
      auto refill_b = [&](int kk) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) fb[kk][nb] = bfrag(br, nb, kk);
        __builtin_amdgcn_s_setprio(0);
      };
      // the fragments read during the previous step (and its flag words) have landed
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
      // unit 0 of sub-step 0 reads registers only: ahead of the barrier
      if (kept(fc, 0, 0)) unit_mfma(0, 0, fa, fb);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(wait_vm(NL));  // stage s1 landed (A(s2) in flight)
      stage_barrier();
      if constexpr (FLAGS) asm volatile("" : "+s"(kwf), "+s"(fcf));
      const uint32_t kb = kbits(kwf);  // A(s3)
      const uint64_t fcnn = fcf;               // MFMA word of s2
      // The buffers of step s0 are free: B(s2) and then A(s3) go there, one
      // load between two units' MFMAs (a burst of loads stalls the wave on
      // the address queue while its MFMAs wait behind them).
      issueB1(s2, bb, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (kept(fc, 0, 1)) unit_mfma(0, 1, fa, fb);
      __builtin_amdgcn_sched_barrier(0);
      issueB1(s2, bb, 1);
      refill_unit(0, 0);
      refill_unit(0, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (kept(fc, 0, 2)) unit_mfma(0, 2, fa, fb);
      __builtin_amdgcn_sched_barrier(0);
      issueB1(s2, bb, 2);
      refill_unit(0, 2);
      __builtin_amdgcn_sched_barrier(0);
      if (kept(fc, 0, 3)) unit_mfma(0, 3, fa, fb);
      __builtin_amdgcn_sched_barrier(0);
      issueB1(s2, bb, 3);
      refill_unit(0, 3);
      refill_b(0);
      const int s4 = nxt(s3 + 1);
      kwf = wl(s4);
      fcf = wc(s3);
      const __amdgpu_buffer_rsrc_t rsA3 = arsrc(s3);
#pragma unroll
      for (int u = 0; u < MB / 2; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if (kept(fc, 1, u)) unit_mfma(1, u, fa, fb);
        __builtin_amdgcn_sched_barrier(0);
        issueA1(rsA3, s3, ab, kb, u);
        refill_unit(1, u);
      }
      refill_b(1);
      fc = fcn;
      fcn = fcnn;
      ab = an;
      bb = bn;
      s0 = s1;
      s1 = s2;
      s2 = s3;
      s3 = s4;
    }
  };
  if (walk_all) run(std::true_type{});
  else if constexpr (FLAGS) {
    if (any) run(std::false_type{});
  }
  // drain the loads of the zero-filled stages past the end before the LDS is
  // handed to an epilogue
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  return any;
}

// Row (A side) of accumulator element r of MFMA block mb, relative to the
// wave's first row: a 16x16 block puts 4 consecutive rows in each lane, the
// four 16-lane groups 4 rows apart.  The lane's column is l & 15.  Tests of
// a row against a per-lane bound are written as the compile-time part
// (mb * 16 + r) against the bound minus the lane part, so no per-element
// row values are kept in registers.
__device__ __forceinline__ int acc_row(int mb, int r, int l) {
  return mb * 16 + (l >> 4) * 4 + r;
}
__device__ __forceinline__ int lane_row(int l) { return (l >> 4) * 4; }

// ---------------------------------------------------------------------------
// Forward: logit tiles -> per-(slab, token) (max, sum exp(a - max)) partials.  Rows of the MFMA tile are vocabulary entries,
// columns are tokens, so each lane owns whole tokens (4 per lane) and folds
// its 32 values of each per tile without shuffles.
// ---------------------------------------------------------------------------
// RAGGED is set only for the launch of the last slab, whose final tile may
// run past V: its rows past V are masked to -inf.  Keeping that code out of
// the main launch keeps its register allocation lean.
template <bool RAGGED>
__global__ __launch_bounds__(NTHREADS) void k_fwd_lse(const u16 *__restrict__ C,
                                                      const u16 *__restrict__ E, int N, int V,
                                                      int D, int TT, int VTr, int vt_base,
                                                      int slab0, int nslab,
                                                      const int64_t *__restrict__ x,
                                                      int64_t ignore_index,
                                                      float *__restrict__ pm,
                                                      float *__restrict__ ps,
                                                      const int64_t *__restrict__ nvalid) {
  __shared__ __attribute__((aligned(16))) u16 lds[PipeF::LDS + BN * 2];  // + target table
  // rows are compacted (valid first): only the token tiles that hold valid
  // rows are numbered, and a tile of ignored rows only has no work
  const int Nv = load_nvalid(nvalid);
  const int TTv = live_tiles(Nv, TT, 8);
  const int G = TTv * nslab;
  if ((int)blockIdx.x >= G) return;
  const int L = xcd_remap(blockIdx.x, G);
  int ls, tt;  // slab within this launch, token tile
  grouped(L, nslab, TTv, ls, tt);
  const int slab = slab0 + ls;  // row of the partials
  const int n0 = tt * BN;
  if (n0 >= Nv) return;
  // this launch's VTr vocabulary tiles from vt_base on, split into nslab slabs
  const int vt0 = vt_base + (int)((int64_t)ls * VTr / nslab);
  const int vt1 = vt_base + (int)((int64_t)(ls + 1) * VTr / nslab);
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave_m(w), wn = wave_n(w);

  const int tok0 = n0 + wn * WCOLS + (l & 15);  // the lane's token of block nb: + 16 nb
  // Each token's target id (-1 if none), in LDS past the operand stages: the
  // fold leaves the target entry out, so the partials are the max and sum
  // over the other entries, and the merge adds the target logit from the
  // indexed dot (fp64) as a softplus.  The target usually dominates the sum;
  // the tile's fp32 accumulation over K = D carries an error of about 1e-6 of
  // its running magnitude, and lse - t in fp32 would cancel when the loss is
  // small.  (Part of the one LDS array: with a second LDS object the compiler
  // can no longer tell the loop's fragment reads from the direct-to-LDS loads
  // in flight and waits for all of them.)
  int *tinfo = reinterpret_cast<int *>(lds + PipeF::LDS);
  if (t < BN) {
    int ti = -1;
    const int n = n0 + t;
    if (n < N) {
      const int64_t xv = x[n];
      if (xv != ignore_index && xv >= 0 && xv < V) ti = (int)xv;
    }
    tinfo[t] = ti;
  }
  __syncthreads();
  float m[NB], s[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = -INFINITY;
    s[nb] = 0.0f;
  }

  const int brows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(E + (int64_t)n0 * D, (int64_t)brows * D * 2);
  f32x4 acc[MB][NB];

  auto rsrcA = [&](int vt) __attribute__((always_inline)) {
    const int m0 = vt * BM;
    return make_rsrc(C + (int64_t)m0 * D, (int64_t)min(BM, V - m0) * D * 2);
  };
  if (vt0 < vt1) mainloop_prologue<PipeF>(rsrcA(vt0), D * 2, rsB, D * 2, D, lds);
  for (int vt = vt0; vt < vt1; ++vt) {
    const int m0 = vt * BM;
    mainloop<PipeF, false, true>(rsrcA(vt), D * 2, rsB, D * 2, D, lds, acc);
    // the next tile's first stages load while this one's epilogue runs
    if (vt + 1 < vt1) mainloop_prologue<PipeF>(rsrcA(vt + 1), D * 2, rsB, D * 2, D, lds);

    const int vbase = m0 + wm * 128;  // first vocabulary row of this wave
    const bool ragged = RAGGED && m0 + BM > V;  // final tile: rows past V are -inf
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // one token's 32 logits of this tile, folded in the accumulators
      // (element r of block mb is row mb * 16 + lane_row(l) + r)
      if (ragged) {
        const int lim = V - vbase - lane_row(l);  // rows from lim on are past V
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mb * 16 + r >= lim) acc[mb][nb][r] = -INFINITY;
      }
      const int ti = tinfo[wn * WCOLS + nb * 16 + (l & 15)];
      const int rel = ti - vbase;  // target row within this wave's 128 rows
      if (__ballot(ti >= 0 && (unsigned)rel < 128u) != 0ull) {  // rare
        const int rl = rel - lane_row(l);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mb * 16 + r == rl) acc[mb][nb][r] = -INFINITY;
      }
      float lm = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) lm = fmaxf(lm, acc[mb][nb][r]);
      if (lm > -INFINITY) {
        const float mn = fmaxf(m[nb], lm);
        const float mL = mn * LOG2E;
        float ts = 0.0f;  // this tile's sum first, then one add into the running sum
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) ts += exp2_fast(fmaf(acc[mb][nb][r], LOG2E, -mL));
        s[nb] = s[nb] * exp2_fast((m[nb] - mn) * LOG2E) + ts;
        m[nb] = mn;
      }
      __builtin_amdgcn_sched_barrier(0);  // keep one token's values live at a time
    }
  }

  // Combine the four 16-lane groups (same tokens, different vocabulary
  // rows), in a fixed order ...
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float mo = __shfl_xor(m[nb], o);
      const float so = __shfl_xor(s[nb], o);
      const float M = fmaxf(m[nb], mo);
      float Ssum = 0.0f;
      if (M > -INFINITY)
        Ssum = s[nb] * exp2_fast((m[nb] - M) * LOG2E) + so * exp2_fast((mo - M) * LOG2E);
      m[nb] = M;
      s[nb] = Ssum;
    }
  }
  // ... then the two waves that share tokens, through LDS.
  __syncthreads();
  float *red = reinterpret_cast<float *>(lds);
  if (wm == 1 && l < 16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = wn * WCOLS + nb * 16 + l;
      red[2 * c] = m[nb];
      red[2 * c + 1] = s[nb];
    }
  }
  __syncthreads();
  if (wm == 0 && l < 16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = wn * WCOLS + nb * 16 + l;
      const float mo = red[2 * c], so = red[2 * c + 1];
      const float M = fmaxf(m[nb], mo);
      float Ssum = 0.0f;
      if (M > -INFINITY)
        Ssum = s[nb] * exp2_fast((m[nb] - M) * LOG2E) + so * exp2_fast((mo - M) * LOG2E);
      const int tok = tok0 + nb * 16;
      if (tok < N) {
        pm[(int64_t)slab * N + tok] = M;
        ps[(int64_t)slab * N + tok] = Ssum;
      }
    }
  }
}

// The target logit t_n = C[x_n] . E_n ("Cut Your Losses" digest, Algorithm 1:
// the indexed matrix multiplication), one wave per token: each lane takes
// 8-element chunks at stride 512 elements, products of the bf16 inputs
// (exact) summed in fp64 in a fixed order, then a fixed butterfly over the
// wave.  fp64 keeps the target logit exact to ~1e-15 relative, so the loss
// formed from it in the merge is limited by the other logits only.  Rows with
// an ignored or out-of-range target are skipped (the merge never reads them).
__global__ __launch_bounds__(256) void k_target(const u16 *__restrict__ C,
                                                const u16 *__restrict__ E,
                                                const int64_t *__restrict__ x, int N, int V, int D,
                                                int64_t ignore_index, double *__restrict__ tlogit) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (n >= N) return;
  const int64_t xv = x[n];
  if (xv == ignore_index || xv < 0 || xv >= V) return;
  const u16 *e = E + (int64_t)n * D;
  const u16 *c = C + xv * (int64_t)D;
  double acc = 0.0;
  for (int d = l * 8; d < D; d += 512) {
    const u32x4 ev = *reinterpret_cast<const u32x4 *>(e + d);
    const u32x4 cv = *reinterpret_cast<const u32x4 *>(c + d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fma((double)bf2f((u16)(ev[j] & 0xffffu)), (double)bf2f((u16)(cv[j] & 0xffffu)), acc);
      acc = fma((double)bf2f((u16)(ev[j] >> 16)), (double)bf2f((u16)(cv[j] >> 16)), acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (l == 0) tlogit[n] = acc;
}

// Fixed-order block reduction of doubles (256 threads).
__device__ double block_sum_256(double v, double *sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  return sh[0];
}

// Row n of the compacted order goes to output row perm[n]; ignored rows get
// lse = loss = 0 without reading the partials (their tiles never ran).
// For a row with a target the partials hold the max M and the sum S of
// exp(a - M) over the other entries (the fold leaves the target out), so with
// z = M + ln S - t the loss is softplus(z) = ln(1 + e^z) and lse = t + loss:
// the same numbers as lse - t ("Cut Your Losses" digest, "The Mathematical
// Decomposition"), formed in fp64 without the cancellation of lse - t when
// the target dominates.  A row whose target lies outside [0, V) gets the lse
// of every entry and a NaN loss.
__global__ __launch_bounds__(256) void k_fwd_merge(const float *__restrict__ pm,
                                                   const float *__restrict__ ps,
                                                   const double *__restrict__ tlogit,
                                                   const int64_t *__restrict__ x,
                                                   const int32_t *__restrict__ perm, int N, int V,
                                                   int S, int64_t ignore_index, int reduction,
                                                   float *__restrict__ loss,
                                                   float *__restrict__ lse,
                                                   double *__restrict__ bsum) {
  __shared__ double sh[256];
  const int n = blockIdx.x * 256 + threadIdx.x;
  double mine = 0.0;
  if (n < N) {
    const int64_t xv = x[n];
    float lo = 0.0f, ls = 0.0f;
    if (xv != ignore_index) {
      float M = -INFINITY;
      for (int k = 0; k < S; ++k) M = fmaxf(M, pm[(int64_t)k * N + n]);
      double Ssum = 0.0;
      if (M > -INFINITY)
        for (int k = 0; k < S; ++k)
          Ssum += (double)ps[(int64_t)k * N + n] * exp((double)pm[(int64_t)k * N + n] - (double)M);
      // ln of the sum over the entries the partials hold (-inf: none)
      const double lsum = Ssum > 0.0 ? (double)M + log(Ssum) : -INFINITY;
      if (xv >= 0 && xv < V) {
        const double t = tlogit[n];
        const double z = lsum - t;
        const double sp = z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));  // 0 when z = -inf
        ls = (float)(t + sp);
        lo = (float)sp;
        mine = sp;
      } else {
        ls = (float)lsum;
        lo = __builtin_nanf("");
        mine = (double)lo;
      }
    }
    const int o = perm[n];
    lse[o] = ls;
    if (reduction == CCE_REDUCTION_NONE) loss[o] = lo;
  }
  if (reduction != CCE_REDUCTION_NONE) {
    const double tot = block_sum_256(mine, sh);
    if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
  }
}

__global__ __launch_bounds__(256) void k_fwd_reduce(const double *__restrict__ bsum, int nblocks,
                                                    const int64_t *__restrict__ nvalid,
                                                    int reduction, float *__restrict__ loss) {
  __shared__ double sh[256];
  double v = 0.0;
  for (int i = threadIdx.x; i < nblocks; i += 256) v += bsum[i];
  const double tot = block_sum_256(v, sh);
  if (threadIdx.x == 0) {
    const int64_t nv = *nvalid;
    loss[0] = (float)(reduction == CCE_REDUCTION_MEAN ? tot / (double)(nv > 0 ? nv : 1) : tot);
  }
}

// Ignored rows removed ahead of the loss ("Cut Your Losses" digest, Table A1:
// dropping ignored tokens before the kernels): a stable partition of the rows,
// perm[0 .. Nv) the valid rows (x != ignore_index) in order, perm[Nv .. N)
// the ignored ones, xc = x[perm], nvalid = Nv.  Every kernel after it works on
// the compacted rows and stops at Nv; the outputs go back through perm.  One
// workgroup: thread t takes rows [t*per, t*per + per), an exclusive scan of
// the per-thread counts gives each thread its place in both halves.  Also
// clears the filter counters and the per-call slots.
__global__ __launch_bounds__(1024) void k_compact(const int64_t *__restrict__ x, int N,
                                                  int64_t ignore_index,
                                                  int32_t *__restrict__ perm,
                                                  int64_t *__restrict__ xc,
                                                  int64_t *__restrict__ nvalid,
                                                  unsigned long long *__restrict__ counter,
                                                  uint32_t *__restrict__ slots, int nslots) {
  for (int i = threadIdx.x; i < nslots; i += 1024) slots[i] = 0u;
  __shared__ int sh[1024];
  const int t = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int r0 = min(N, t * per), r1 = min(N, r0 + per);
  int c = 0;
  for (int n = r0; n < r1; ++n) c += (x[n] != ignore_index) ? 1 : 0;
  // inclusive scan of the counts (Hillis-Steele over the 1024 threads)
  sh[t] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = t >= o ? sh[t - o] : 0;
    __syncthreads();
    sh[t] += v;
    __syncthreads();
  }
  const int nv = sh[1023];
  int pv = sh[t] - c;      // valid rows before this thread's range
  int pi = nv + r0 - pv;   // ... and where its ignored rows go
  for (int n = r0; n < r1; ++n) {
    const int64_t xv = x[n];
    const int o = (xv != ignore_index) ? pv++ : pi++;
    perm[o] = n;
    xc[o] = xv;
  }
  if (t == 0) *nvalid = nv;
  if (counter && t < NCOUNT) counter[t] = 0ull;
}

// Ec[i] = E[perm[i]] for the valid rows, zero rows after them: the ignored
// rows' values never enter any arithmetic (a tile that straddles the valid
// count, the scale of E, its transpose), whatever they hold.  16 bytes per
// thread and step.
__global__ __launch_bounds__(256) void k_gather_rows(const u16 *__restrict__ E,
                                                     const int32_t *__restrict__ perm, int N,
                                                     int D, const int64_t *__restrict__ nvalid,
                                                     u16 *__restrict__ Ec) {
  const int cpr = D / 8;  // 16-byte chunks per row
  const int64_t total = (int64_t)N * cpr;
  const int64_t nv = *nvalid;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / cpr;
    const int c = (int)(i - row * cpr);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < nv) v = *reinterpret_cast<const u32x4 *>(E + (int64_t)perm[row] * D + c * 8);
    *reinterpret_cast<u32x4 *>(Ec + row * D + c * 8) = v;
  }
}

// Per-row backward state of the compacted row n (original row perm[n]):
// lse*log2(e), the upstream scale, the target.  The ignored rows (the end of
// the compacted order) get exactly zero dE rows here; no later kernel writes
// them.
__global__ __launch_bounds__(256) void k_bwd_rows(const int64_t *__restrict__ xc,
                                                  const int32_t *__restrict__ perm,
                                                  const float *__restrict__ lse,
                                                  const float *__restrict__ grad, int N, int Npad,
                                                  int V, int D, int64_t ignore_index,
                                                  int reduction,
                                                  const int64_t *__restrict__ nvalid,
                                                  const double *__restrict__ tlogit,
                                                  RowInfo *__restrict__ ri,
                                                  float *__restrict__ srow,
                                                  uint32_t *__restrict__ sigma,
                                                  u16 *__restrict__ dE,
                                                  const int32_t *__restrict__ vpos) {
  __shared__ int zrow[256];
  const int n = blockIdx.x * 256 + threadIdx.x;
  RowInfo r = {INFINITY, 0.0f, -1, 0};
  float sn = 0.0f;  // the row's upstream scale
  int zr = -1;
  if (n < N) {
    const int64_t xv = xc[n];
    const int o = perm[n];
    if (xv != ignore_index) {
      float sc;
      if (reduction == CCE_REDUCTION_NONE) {
        sc = grad[o];
      } else if (reduction == CCE_REDUCTION_SUM) {
        sc = grad[0];
      } else {
        const int64_t nv = *nvalid;
        sc = (float)((double)grad[0] / (double)(nv > 0 ? nv : 1));
      }
      // a target outside [0, V) is treated like an ignored row here; with a
      // vocabulary order the target is its entry's position (vpos), and an
      // entry the order does not hold (vpos < 0) leaves the row without G
      const int32_t tg = (xv >= 0 && xv < V) ? (vpos ? vpos[xv] : (int32_t)xv) : -1;
      if (tg >= 0) {
        r.lse2 = lse[o] * LOG2E;
        // p_t - 1 from the exact target logit: when the target dominates,
        // 1 - p_t is far below the fp32 error of the tile's logit (~1e-6 of
        // its magnitude), and only the rounding of the given lse is left
        r.gt = (float)expm1(tlogit[n] - (double)lse[o]);
        r.live = 1;
        r.tgt = tg;
        sn = sc;
        atomicMax(sigma, __float_as_uint(fabsf(sc)));
      }
    } else {
      zr = o;
    }
  }
  if (n < Npad) {
    ri[n] = r;
    srow[n] = sn;
  }
  zrow[threadIdx.x] = zr;
  // zero the dE rows of this block's ignored rows, the whole block per row
  if (__syncthreads_count(zr >= 0) == 0) return;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 256; ++i) {
    const int o = zrow[i];
    if (o < 0) continue;
    for (int c = threadIdx.x; c < D / 8; c += 256)
      *reinterpret_cast<u32x4 *>(dE + (int64_t)o * D + c * 8) = z;
  }
}

// Backward step 1 for one vocabulary chunk: recompute the 256x256 logit tile,
// G = exp(A - lse) - onehot, the 32x32-unit filter by wavefront ballot, fp16;
// write G-hat once, as [n][v] in 8-entry blocks (Gnv: dE reads it as it is,
// dC with transposing LDS reads), for the units either contraction keeps, and
// the unit flags in the two orders the contractions read.  Each contraction
// has its own threshold ("Cut Your Losses" digest, "Numerical Stability
// Variants": FullC leaves dC unfiltered, FullE dE); a threshold of 0 keeps
// every unit.  Flag maps:
//   map2[((vu >> 2) * NU + nu) * 4 + (vu & 3)]   (dC: 4 vocab units per word)
//   map3[((nu >> 2) * VU + vu) * 4 + (nu & 3)]   (dE: 4 token units per word)
struct GradArgs {
  const u16 *C, *E;
  const RowInfo *ri;
  int N, V, D, v_start, chunk_len, NTt, VTt;
  float eps_dE, eps_dC;  // filter thresholds of dE and dC
  // G-hat element (n, v) at ((v / 8) * rows_nv + n) * 8 + v % 8, n within the
  // token block, rows_nv = the block's padded rows: each store fills half of
  // a 16-byte cell; a 64-token run of one 8-entry block is 1 KiB contiguous
  // (one load of dC's operand).
  u16 *Gnv;
  int rows_nv;
  unsigned long long *counter;
  uint8_t *map2, *map3;
  int NU, VU;
  const int64_t *nvalid;  // compacted rows: tiles past it have no work
  // vocabulary order ("Cut Your Losses" digest, "Vocabulary Sorting"): chunk
  // row v is entry vorder[v_start + v] (the sorted launches only)
  const int32_t *vorder;
  int row0;  // the token block's first compacted row (E, ri and Gnv start there)
};

// LDS of the fused backward step: the operand stages of the main loops.
constexpr int LDS_BWD = LDS_MAIN;

template <bool SORTED>
__device__ __forceinline__ void grad_tile(const GradArgs &a, int L, int NTv, u16 *lds) {
  const u16 *__restrict__ C = a.C;
  const u16 *__restrict__ E = a.E;
  const RowInfo *__restrict__ ri = a.ri;
  const int N = a.N, V = a.V, D = a.D, v_start = a.v_start, chunk_len = a.chunk_len;
  const int rows_nv = a.rows_nv, NU = a.NU, VU = a.VU;
  const float eps_dE = a.eps_dE, eps_dC = a.eps_dC;
  u16 *__restrict__ Gnv = a.Gnv;
  uint8_t *__restrict__ map2 = a.map2;
  uint8_t *__restrict__ map3 = a.map3;
  int vt, ntile;
  grouped(L, a.VTt, NTv, vt, ntile);  // NTv: token tiles with valid rows
  const int m0 = vt * BM;  // chunk-local vocabulary row
  const int n0 = ntile * BN;
  const int Nv = max(0, load_nvalid(a.nvalid) - a.row0);  // valid rows of the block
  // Tiles of ignored rows only are skipped: their G is zero, dC reads no
  // column past the last tile that runs and dE has no tile there.
  if (n0 >= Nv) return;
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave_m(w), wn = wave_n(w);

  const int arows = max(0, min(BM, chunk_len - m0));
  const int brows = max(0, min(BN, N - n0));
  const __amdgpu_buffer_rsrc_t rsB =
      make_rsrc(E + (int64_t)min(n0, max(N - 1, 0)) * D, (int64_t)brows * D * 2);
  f32x4 acc[MB][NB];
  if constexpr (SORTED) {
    // the tile's C rows are gathered from anywhere in C (V * D * 2 bytes fit
    // a buffer offset: checked on the host)
    const __amdgpu_buffer_rsrc_t rsC = make_rsrc(C, (int64_t)V * D * 2);
    mainloop_sp<false, false, ALR, false, true>(rsC, D * 2, rsB, D * 2, D, lds, acc, nullptr, 0,
                                                nullptr, false, nullptr, a.vorder + v_start + m0,
                                                arows, V);
  } else {
    const __amdgpu_buffer_rsrc_t rsA =
        make_rsrc(C + (int64_t)(v_start + m0) * D, (int64_t)arows * D * 2);
    mainloop_sp<false, false, ALR>(rsA, D * 2, rsB, D * 2, D, lds, acc);
  }

  __syncthreads();  // every wave is done reading the operand stages

  RowInfo rinf[NB];
  int tok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    tok[nb] = n0 + wn * WCOLS + nb * 16 + (l & 15);
    rinf[nb] = ri[tok[nb]];  // ri has Npad entries
  }
  const int vloc = m0 + wm * 128;  // chunk-local first row of this wave
  // Rows whose G is not computed carry lse2 = +inf, so their exp2 is exactly
  // 0 with no per-element test.  Only the last tile of the last chunk has rows
  // past the chunk, and only where some lane's target falls in this wave's 128
  // rows does an element need the one-hot term; elsewhere every G is >= 0 and
  // the filter test is one compare of the maximum.
  const bool ragged = m0 + BM > chunk_len;
  int trel[NB];   // target row relative to the wave's first row
  bool thit[NB];  // some lane's target is in the wave's rows (wave-uniform)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    trel[nb] = rinf[nb].tgt - (v_start + vloc);
    thit[nb] = __ballot(rinf[nb].tgt >= 0 && (unsigned)trel[nb] < 128u) != 0ull;
  }
  int skipped = 0;  // units dropped from either contraction
  // bit u * CU + c: unit kept for dE ([n][v]) / for dC ([v][n]); wave-uniform
  uint32_t keptE = 0, keptC = 0;
  // A 32x32 unit (row unit u, column unit c) is MFMA blocks 2u, 2u + 1 by
  // 2c, 2c + 1: each lane holds 4 values of each of the four blocks.
#pragma unroll
  for (int u = 0; u < MB / 2; ++u) {
#pragma unroll
    for (int c = 0; c < CU; ++c) {
      float g[2][2][4];  // [row block][column block][element]
      float mg = 0.0f;   // the lane's largest |G| in the unit
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = 2 * c + j;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int mb = 2 * u + i;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            g[i][j][r] = exp2_fast(fmaf(acc[mb][nb][r], LOG2E, -rinf[nb].lse2));
          if (ragged) {
            const int lim = chunk_len - vloc - lane_row(l);  // rows >= lim are past the chunk
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (mb * 16 + r >= lim) g[i][j][r] = 0.0f;
          }
        }
        if (thit[nb]) {
          const int rl = trel[nb] - lane_row(l);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if ((2 * u + i) * 16 + r == rl) g[i][j][r] = rinf[nb].gt;
              mg = fmaxf(mg, fabsf(g[i][j][r]));
            }
        } else {  // no one-hot term: every G is >= 0
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) mg = fmaxf(mg, g[i][j][r]);
        }
      }
      const bool kE = __ballot(mg >= eps_dE) != 0ull;
      const bool kC = __ballot(mg >= eps_dC) != 0ull;
      if (!(kE && kC)) {
        const int vu = v_start + vloc + u * 32;
        const int nu = n0 + wn * WCOLS + c * 32;
        if (vu < V && nu < Nv) ++skipped;
      }
      if (kE || kC) {
        keptE |= (uint32_t)kE << (u * CU + c);
        keptC |= (uint32_t)kC << (u * CU + c);
        // for each block this lane holds 4 consecutive vocabulary rows of its
        // token: 8 bytes, half of a 16-byte cell
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nb = 2 * c + j;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int v = m0 + wm * 128 + acc_row(2 * u + i, 0, l);
            u32x2 pk;
            pk.x = (uint32_t)f2h(GSCALE * g[i][j][0]) | ((uint32_t)f2h(GSCALE * g[i][j][1]) << 16);
            pk.y = (uint32_t)f2h(GSCALE * g[i][j][2]) | ((uint32_t)f2h(GSCALE * g[i][j][3]) << 16);
            *reinterpret_cast<u32x2 *>(Gnv + ((int64_t)(v >> 3) * rows_nv + tok[nb]) * 8 +
                                       (v & 7)) = pk;
          }
        }
      }
    }
  }

  // Unit flags, in the two orders the contractions read.  Filtered units are
  // never written: their flags keep every reader off them.
  if (l < 4 * CU) {
    const int u = l / CU, c = l % CU;
    const uint8_t kc = (uint8_t)((keptC >> (u * CU + c)) & 1u);
    const uint8_t ke = (uint8_t)((keptE >> (u * CU + c)) & 1u);
    const int vu = (m0 + wm * 128) / UNIT + u, nu = (n0 + wn * WCOLS) / UNIT + c;
    map2[((int64_t)(vu >> 2) * NU + nu) * 4 + (vu & 3)] = kc;
    map3[((int64_t)(nu >> 2) * VU + vu) * 4 + (nu & 3)] = ke;
  }

  // Units dropped: one atomic add per workgroup, into one of NCOUNT counters
  // (a single counter serialised thousands of adds per launch).
  uint32_t *cnt_lds = reinterpret_cast<uint32_t *>(lds);  // the stages are done with
  if (l == 0) cnt_lds[w] = (uint32_t)skipped;
  __syncthreads();
  if (t == 0) {
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) tot += cnt_lds[i];
    if (tot) atomicAdd(a.counter + (blockIdx.x % NCOUNT), (unsigned long long)tot);
  }
}

// One pass of a tile's sums into its fp32 accumulator, kept in register
// order: every lane's 4 values of an MFMA block are 16 contiguous bytes (each
// wave's slice of a block one contiguous 1 KiB run); tacc is the lane's first
// value.  scale(mb) multiplies block row mb's sums; first: the accumulator is
// not read; last: the total goes to store(mb, nb, v) instead of back.  The
// earlier passes' sums come back in batches of two block rows (8 accesses in
// flight), each batch requested before the previous one is added and stored
// back: in program order no load follows a store it could be taken to depend
// on, so the waits are partial (one access at a time, each behind its own
// store, left the latency exposed 32 times).
template <typename Scale, typename Store>
__device__ __forceinline__ void acc_pass(float *__restrict__ tacc, const f32x4 (&acc)[MB][NB],
                                         bool first, bool last, Scale scale, Store store) {
  constexpr int BR = 2, NBATCH = MB / BR;
  u32x4 prev[2][BR][NB];  // [batch parity][block row][block column]
  auto load_batch = [&](int bt, u32x4 (&dst)[BR][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < BR; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        dst[i][nb] =
            *reinterpret_cast<const u32x4 *>(tacc + (int64_t)((bt * BR + i) * NB + nb) * 64 * 4);
  };
  if (!first) load_batch(0, prev[0]);
#pragma unroll
  for (int bt = 0; bt < NBATCH; ++bt) {
    if (!first && bt + 1 < NBATCH) load_batch(bt + 1, prev[(bt + 1) & 1]);
#pragma unroll
    for (int i = 0; i < BR; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int mb = bt * BR + i;
      f32x4 v = acc[mb][nb] * scale(mb);
      if (!first) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += __uint_as_float(prev[bt & 1][i][nb][e]);
      }
      if (last) {
        store(mb, nb, v);
      } else {
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = __float_as_uint(v[e]);
        *reinterpret_cast<u32x4 *>(tacc + (int64_t)(mb * NB + nb) * 64 * 4) = u;
      }
    }
  }
}

// Backward step 2: dC[v_start + v][d] = sum_n G-hat[v][n] E[n][d] for the
// chunk.  Each workgroup owns a disjoint 256-row vocabulary panel and sums
// over the tokens in registers, no atomics: all of them at once (one bf16
// write), or, when the backward takes the tokens in blocks, one block per
// launch, the blocks' sums added in block order into an fp32 accumulator
// (mode bit 0: first block, no read of it; bit 1: last block, cast to bf16
// into dC).
struct DcArgs {
  const u16 *Gnv;  // G-hat in 8-entry blocks (see GradArgs), read transposed
  int rows_nv;
  const u16 *Et;  // s_n E_n (scaled fp16) in 8-token blocks: (d, n) at ((n / 8) * Dpad + d) * 8 + n % 8
  int Kn, chunk_len, v_start, D, DT, VTt;
  u16 *dC;
  const uint32_t *sigma_bits, *amaxE;
  const uint8_t *map2;
  int NU;
  const int64_t *nvalid;
  int filtered;  // dC takes the filtered G-hat (some units may be dropped)
  const int32_t *vorder;  // sorted launches: chunk row v is dC row vorder[v_start + v]
  int V;
  int row0;      // the token block's first compacted row (Gnv, Et and K start there)
  float *dCacc;  // the chunk's fp32 sums over the earlier blocks (mode != 3)
  int mode;
};

template <bool SORTED>
__device__ __forceinline__ void dc_tile(const DcArgs &a, int L, u16 *lds) {
  const u16 *__restrict__ Gnv = a.Gnv;
  const u16 *__restrict__ Et = a.Et;
  const int rows_nv = a.rows_nv, Kn = a.Kn, chunk_len = a.chunk_len;
  const int v_start = a.v_start, D = a.D, DT = a.DT, NU = a.NU;
  u16 *__restrict__ dC = a.dC;
  const uint8_t *__restrict__ map2 = a.map2;
  int vt, dt;
  strips(L, a.VTt, DT, vt, dt);
  const int m0 = vt * BM, n0 = dt * BN;
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave_m(w), wn = wave_n(w);
  // the tile's vocabulary units m0/32 .. +7 form map2 groups m0/128, +1
  const uint64_t *fw = reinterpret_cast<const uint64_t *>(map2) + (int64_t)(m0 / 128) * (NU / 2);
  // K = the token columns of the G-hat tiles that ran (whole 256-token tiles
  // of the compacted rows)
  const int Nv = max(0, load_nvalid(a.nvalid) - a.row0);  // valid rows of the block
  const int Kr = min(Kn, (Nv + BN - 1) / BN * BN);
  // a block between the first and the last with no valid rows adds nothing
  // (the first writes the accumulator, the last casts it, whatever their rows)
  if (Kr == 0 && a.mode == 0) return;
  const uint32_t sigma_bits = ld_const_u32(a.sigma_bits), amax_bits = ld_const_u32(a.amaxE);
  f32x4 acc[MB][NB];
  const __amdgpu_buffer_rsrc_t none = make_rsrc(Et, 0);  // both operands use per-step descriptors
  const bool walked =
      mainloop_sp<true, true, ALT, true>(none, rows_nv * 16, none, DT * BN * 16, Kr, lds, acc, fw,
                                         NU / 2, Gnv + (int64_t)(m0 / 8) * rows_nv * 8,
                                         a.filtered != 0, Et + (int64_t)n0 * 8);
  // likewise a middle block whose units were all filtered
  if (!walked && a.mode == 0) return;
  // 1 / (GSCALE * scale(s E)), exact: a power of two (the E operand holds
  // s_n E_n scaled by the power of two of sigma * max|E|, sigma = max |s_n|)
  const float f = (1.0f / GSCALE) * pow2_recip_f(__uint_as_float(sigma_bits) * bf2f((u16)amax_bits));
  const int mode = a.mode;
  // sorted launches: the tile's 256 output rows, staged in LDS once the loop
  // is done with it (-1: no row)
  const int32_t *rowid = reinterpret_cast<const int32_t *>(lds);
  if constexpr (SORTED) {
    if (mode & 2) {
      __syncthreads();
      if (t < BM) {
        const int g = m0 + t < chunk_len ? a.vorder[v_start + m0 + t] : -1;
        reinterpret_cast<int32_t *>(lds)[t] = (g >= 0 && g < a.V) ? g : -1;
      }
      __syncthreads();
    }
  }
  auto store = [&](int mb, int nb, f32x4 v) __attribute__((always_inline)) {
    const int d = n0 + wn * WCOLS + nb * 16 + (l & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (SORTED) {
        const int g = rowid[wm * 128 + acc_row(mb, r, l)];
        if (g >= 0 && d < D) dC[(int64_t)g * D + d] = f2bf(v[r]);
      } else {
        const int v_ = m0 + wm * 128 + acc_row(mb, r, l);
        if (v_ < chunk_len && d < D) dC[(int64_t)(v_start + v_) * D + d] = f2bf(v[r]);
      }
    }
  };
  if (mode == 3) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store(mb, nb, acc[mb][nb] * f);
  } else {
    acc_pass(a.dCacc + (((int64_t)L * NWAVES + w) * MB * NB * 64 + l) * 4, acc, (mode & 1) != 0,
             (mode & 2) != 0, [&](int) __attribute__((always_inline)) { return f32x4{f, f, f, f}; },
             store);
  }
}

// Backward step 3: dE[n][d] (+)= sum_v G-hat[n][v] C[v_start + v][d] for the
// chunk.  The chunks are the split-K slices of the vocabulary sum, added in
// chunk order into an fp32 accumulator.  mode bit 0: first chunk (no read of
// the accumulator); bit 1: last chunk (cast to bf16 into dE).
struct DeArgs {
  const u16 *Gnv;  // 8-entry blocks (see GradArgs)
  int rows_nv;
  const u16 *Ct;  // the chunk's scaled fp16 C in 8-row blocks: (d, v) at ((v / 8) * Dpad + d) * 8 + v % 8
  int Kv, N, D, DT, MTt, mode;
  float *dEacc;
  u16 *dE;
  const float *srow;  // s_n of each compacted row (Npad entries)
  const uint32_t *amaxC;
  const uint8_t *map3;
  int VU;
  const int64_t *nvalid;
  const int32_t *perm;  // compacted row -> output row
  int filtered;         // dE takes the filtered G-hat (some units may be dropped)
  // Split over the chunk's vocabulary rows (few dE tiles, small N): part p
  // of every tile takes rows [p * kpart, (p + 1) * kpart) of each chunk and
  // keeps its own accumulator (part_stride floats apart); k_de_final adds
  // the parts.  nparts == 1: the whole chunk, one accumulator.
  int kpart, nparts;
  int64_t part_stride;
  int row0;  // the token block's first compacted row (Gnv, dEacc, srow and perm start there)
};

__device__ __forceinline__ void de_tile(const DeArgs &a, int L, int MTv, int part, u16 *lds) {
  const u16 *__restrict__ Gnv = a.Gnv;
  const u16 *__restrict__ Ct = a.Ct;
  const int rows_nv = a.rows_nv, D = a.D, DT = a.DT;
  const int mode = a.mode, VU = a.VU;
  const int k0 = part * a.kpart;                    // first chunk row of this part
  const int Kv = min(a.Kv - k0, a.kpart);           // > 0: parts are dealt only where rows are
  float *__restrict__ dEacc = a.dEacc + part * a.part_stride;
  u16 *__restrict__ dE = a.dE;
  const uint8_t *__restrict__ map3 = a.map3;
  int mtile, dt;
  strips(L, MTv, DT, mtile, dt);  // MTv: token tiles with valid rows
  const int m0 = mtile * BM, n0 = dt * BN;
  // compacted rows: a tile of ignored rows only has no work (k_bwd_rows
  // zeroes their dE rows)
  const int Nv = max(0, load_nvalid(a.nvalid) - a.row0);  // valid rows of the block
  if (m0 >= Nv) return;
  const int32_t *__restrict__ perm = a.perm;
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave_m(w), wn = wave_n(w);
  // one flag word per 64-row K-step; G-hat in 8-row k blocks of rows_nv rows
  const uint64_t *fw =
      reinterpret_cast<const uint64_t *>(map3) + (int64_t)(m0 / 128) * (VU / 2) + k0 / 64;
  const uint32_t amax_bits = ld_const_u32(a.amaxC);
  f32x4 acc[MB][NB];
  const int Dpad = DT * BN;
  const __amdgpu_buffer_rsrc_t none = make_rsrc(Ct, 0);  // both operands use per-step descriptors
  const bool walked =
      mainloop_sp<true, true, ALK, true>(none, rows_nv * 16, none, Dpad * 16, Kv, lds, acc, fw,
                                         VU / 2,
                                         Gnv + (int64_t)m0 * 8 + (int64_t)(k0 / 8) * rows_nv * 8,
                                         a.filtered != 0, Ct + ((int64_t)(k0 / 8) * Dpad + n0) * 8);
  const bool first = mode & 1, last = mode & 2;
  // a chunk whose units of this tile were all filtered adds nothing: the
  // sums stay as they are, unless this chunk writes them first or casts them
  if (!walked && !first && !last) return;
  // 1 / (GSCALE * scale(C)), exact (a power of two), times the row's s_n
  const float f = (1.0f / GSCALE) * pow2_recip(amax_bits);
  // s_n of the lane's 4 rows of block mb (srow has Npad entries)
  const float *srow_l = a.srow + m0 + wm * 128 + lane_row(l);
  // the output rows of the lane's 4 rows per block, loaded at once (16 bytes
  // per block; perm has Npad entries) rather than one dependent load per store
  u32x4 prow[MB];
  if (last) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      prow[mb] = *reinterpret_cast<const u32x4 *>(perm + m0 + wm * 128 + mb * 16 + lane_row(l));
  }
  acc_pass(
      dEacc + (((int64_t)L * NWAVES + w) * MB * NB * 64 + l) * 4, acc, first, last,
      [&](int mb) __attribute__((always_inline)) {
        return *reinterpret_cast<const f32x4 *>(srow_l + mb * 16) * f;
      },
      [&](int mb, int nb, f32x4 v) __attribute__((always_inline)) {
        const int d = n0 + wn * WCOLS + nb * 16 + (l & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = m0 + wm * 128 + acc_row(mb, r, l);
          if (n < Nv && d < D) dE[(int64_t)(int)prow[mb][r] * D + d] = f2bf(v[r]);
        }
      });
}

// Transpose role: the B operand of dE for a chunk, Ct(d, v) =
// fp16(C[v_start + v][d] * pow2_scale(amax)) in 8-entry blocks along v
// ((v / 8) * Dpad + d) * 8 + v % 8, zero-padded to Dpad x cpad: dE brings
// 64 consecutive d of one block (1 KiB contiguous) per load.  One workgroup
// converts a 256 x 256 block: all of it is read into LDS at once (16 loads
// in flight per thread), then each wave writes 64 consecutive d x 8
// consecutive v, 1 KiB contiguous (LDS reads of one row of 64 d values per
// instruction: no bank conflicts).
struct TrArgs {
  const u16 *C;
  int chunk_len, D, v_start;
  u16 *Ct;
  int DT;
  const uint32_t *amax;
  const int32_t *vorder;  // sorted launches: chunk row v is C row vorder[v_start + v]
  int V;
};

template <bool SORTED>
__device__ __forceinline__ void tr_tile(const TrArgs &a, int L, u16 *lds) {
  const int vt = L / a.DT, dt = L % a.DT;
  const int v0 = vt * BM, d0 = dt * BN;
  const float sc = pow2_scale(*a.amax);
  const int t = threadIdx.x;
  constexpr int PER = BM * BN / 8 / NTHREADS;  // 16-byte chunks per thread
  u32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int id = t + NTHREADS * i;
    const int row = id >> 5, c = id & 31;  // 32 chunks per 256-wide row
    const int r = v0 + row, col = d0 + c * 8;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (r < a.chunk_len && col < a.D) {
      int64_t src = a.v_start + r;
      if constexpr (SORTED) src = a.vorder[a.v_start + r];
      if (!SORTED || (src >= 0 && src < a.V))
        v[i] = *reinterpret_cast<const u32x4 *>(a.C + src * a.D + col);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int id = t + NTHREADS * i;
    *reinterpret_cast<u32x4 *>(lds + (id >> 5) * TR_STRIDE + (id & 31) * 8) = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int id = t + NTHREADS * i;
    const int drow = id & (BN - 1), vg = id >> 8;  // d row, group of 8 v
    u16 e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = f2h(bf2f(lds[(vg * 8 + j) * TR_STRIDE + drow]) * sc);
    u32x4 o;
    o.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    o.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    o.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    o.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<u32x4 *>(a.Ct + ((int64_t)(v0 / 8 + vg) * (a.DT * BN) + d0 + drow) * 8) = o;
  }
}

// One launch of the backward: the dE and dC tiles of one (chunk, token block)
// pair (reading one G-hat buffer and C^T copy), then the G-hat tiles of the
// next pair and, at a chunk's first block, the transpose of its C rows
// (writing the other copies), in that order of workgroup ids: longest tiles
// first.  A dE tile's K is the chunk (or its part), a dC tile's the block's
// tokens, so dcfirst (set when the tokens are more) puts the dC tiles ahead
// of the dE tiles; a G-hat tile's K is D, a transpose tile has none.  The roles are independent, so the short G-hat
// and transpose tiles fill the CUs the contraction tiles leave idle at the
// end of their last round.  Each contraction role numbers its tiles
// XCD-aware within its own segment (segments are padded to multiples of 8
// workgroups).
template <bool SORTED>
__global__ __launch_bounds__(NTHREADS) void k_bwd_step(DcArgs dc, int nC, int nCp, DeArgs de, int nE,
                                                      int nEp, GradArgs gr, int nG, int nGp,
                                                      TrArgs tr, int nT, int dcfirst,
                                                      const int64_t *__restrict__ nvalid) {
  __shared__ __attribute__((aligned(16))) u16 lds[LDS_BWD];
  int b = blockIdx.x;
  // The dE and G-hat segments are sized for every row; only the tiles of the
  // token tiles that hold valid (compacted) rows are numbered (live_tiles).
  const int Nv = load_nvalid(nvalid);
  const int bE = dcfirst ? b - nCp : b, bC = dcfirst ? b : b - nEp;
  if (bE >= 0 && bE < nEp) {
    const int MTv = live_tiles(max(0, Nv - de.row0), de.MTt, 4);
    const int nEv = min(nE, MTv * de.DT), tot = nEv * de.nparts, totp = (tot + 7) & ~7;
    if (bE < totp) {
      const int L = xcd_remap(bE, totp);
      if (L < tot) de_tile(de, L % nEv, MTv, L / nEv, lds);
    }
    return;
  }
  if (bC >= 0 && bC < nCp) {
    const int L = xcd_remap(bC, nCp);
    if (L < nC) dc_tile<SORTED>(dc, L, lds);
    return;
  }
  b -= nEp + nCp;
  if (b < nGp) {
    const int NTv = live_tiles(max(0, Nv - gr.row0), gr.NTt, 8);
    const int nGv = min(nG, gr.VTt * NTv), nGvp = (nGv + 7) & ~7;
    if (b < nGvp) {
      const int L = xcd_remap(b, nGvp);
      if (L < nGv) grad_tile<SORTED>(gr, L, NTv, lds);
    }
    return;
  }
  b -= nGp;
  if (b < nT) tr_tile<SORTED>(tr, b, lds);
}

// *amax = max over a bf16 array of |value| bits (order-independent max).
// dE of a split backward: the parts' fp32 sums added in part order and cast
// to bf16 into the output rows.  One thread per 16-byte accumulator cell: the
// cell's tile, wave, block and lane give its 4 (row, column) positions the
// way de_tile laid them out.
__global__ __launch_bounds__(256) void k_de_final(const float *__restrict__ dEacc,
                                                  int64_t part_stride, int nparts, int nE, int MTt,
                                                  int DT, int D, const int64_t *__restrict__ nvalid,
                                                  const int32_t *__restrict__ perm,
                                                  u16 *__restrict__ dE) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int Nv = load_nvalid(nvalid);
  const int MTv = live_tiles(Nv, MTt, 4);
  const int nEv = min(nE, MTv * DT);
  constexpr int CELLS = MB * NB * 64;  // per wave
  const int L = (int)(q / ((int64_t)NWAVES * CELLS));
  if (L >= nEv) return;
  const int rem = (int)(q % ((int64_t)NWAVES * CELLS));
  const int w = rem / CELLS, j = (rem % CELLS) / 64, l = rem % 64;
  const int mb = j / NB, nb = j % NB;
  int mtile, dt;
  strips(L, MTv, DT, mtile, dt);
  const int m0 = mtile * BM, n0 = dt * BN;
  const int d = n0 + wave_n(w) * WCOLS + nb * 16 + (l & 15);
  f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int p = 0; p < nparts; ++p) {
    const f32x4 u = *reinterpret_cast<const f32x4 *>(dEacc + p * part_stride + q * 4);
    v += u;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = m0 + wave_m(w) * 128 + acc_row(mb, r, l);
    if (n < Nv && d < D) dE[(int64_t)perm[n] * D + d] = f2bf(v[r]);
  }
}

__global__ __launch_bounds__(256) void k_amax(const u16 *__restrict__ in, int64_t count8,
                                              uint32_t *__restrict__ amax) {
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count8;
       i += (int64_t)gridDim.x * 256) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(in + i * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = max(m, v[j] & 0x7fffu);
      m = max(m, (v[j] >> 16) & 0x7fffu);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (m) atomicMax(amax, m);  // one atomic per workgroup
  }
}

// The dC operand: out(c, r) = fp16(s_r in[r][c] * scale) in 8-entry blocks
// along r, ((r / 8) * Cpad + c) * 8 + r % 8 (Cpad = 64 * gridDim.y), zero
// padded, with s_r the row's upstream scale and scale the power of two that
// maps sigma * max|in| (sigma = max |s_r|) into [2^13, 2^14): dC brings 64
// consecutive c of one block (1 KiB contiguous) per load.  Rows whose s_r is
// far below sigma contribute proportionally little to dC.
__global__ __launch_bounds__(256) void k_transpose(const u16 *__restrict__ in, int R, int Ccols,
                                                   int ld_in, u16 *__restrict__ out,
                                                   const uint32_t *__restrict__ amax,
                                                   const float *__restrict__ srow,
                                                   const uint32_t *__restrict__ sigma) {
  const float sc = pow2_scale_f(__uint_as_float(*sigma) * bf2f((u16)*amax));
  __shared__ __attribute__((aligned(16))) u16 tile[64 * 72];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = t + 256 * i;
    const int row = id >> 3, c = id & 7;
    const int r = r0 + row, col = c0 + c * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && col < Ccols) {
      const u32x4 b = *reinterpret_cast<const u32x4 *>(in + (int64_t)r * ld_in + col);
      const float f = srow[r] * sc;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (uint32_t)f2h(bf2f((u16)(b[j] & 0xffffu)) * f) |
               ((uint32_t)f2h(bf2f((u16)(b[j] >> 16)) * f) << 16);
    }
    *reinterpret_cast<u32x4 *>(tile + row * 72 + c * 8) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = t + 256 * i;
    const int orow = id & 63, oc = id >> 6;  // 64 consecutive c of one block of 8 r
    u16 e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = tile[(oc * 8 + j) * 72 + orow];
    u32x4 v;
    v.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    v.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    v.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    v.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<u32x4 *>(out + ((int64_t)(r0 / 8 + oc) * (64 * gridDim.y) + c0 + orow) * 8) = v;
  }
}

__global__ void k_stats(const unsigned long long *__restrict__ counter,
                        const int64_t *__restrict__ nvalid, int64_t V, int on,
                        cce_filter_stats *__restrict__ st) {
  if (threadIdx.x == 0) {
    // units are cut from the compacted (valid) rows
    st->units_total = (*nvalid + UNIT - 1) / UNIT * ((V + UNIT - 1) / UNIT);
    int64_t skipped = 0;
    for (int i = 0; i < NCOUNT; ++i) skipped += (int64_t)counter[i];
    st->units_skipped = on ? skipped : 0;
    st->unit_rows = UNIT;
    st->unit_cols = UNIT;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t align256(size_t a) { return (a + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Vocabulary order ("Cut Your Losses" digest, "Vocabulary Sorting"): each
// entry's logit averaged over the valid tokens, (1/N_v) sum_n C[v] . E[n] =
// C[v] . mean_n E[n], and the entries sorted by it, largest first, equal
// averages by id.  The digest gathers the sums inside the forward's tiles;
// here the mean row of E is formed first, so the averages cost one pass over
// C.  The sort is a bitonic sort of 64-bit keys (order key of the average,
// entry id): every key is distinct, so the order is fully determined.
// ---------------------------------------------------------------------------
constexpr int VO_RB = 256;       // most row blocks of the mean
constexpr int VO_LOCAL = 4096;   // keys sorted per workgroup in LDS
constexpr int VO_LTHREADS = 1024;  // threads of that workgroup (two key pairs each)

// sums of E over the valid rows of row block blockIdx.y, one column per
// thread; thread 0 of column block 0 counts the block's valid rows
__global__ __launch_bounds__(256) void k_vo_rowsum(const u16 *__restrict__ E,
                                                   const int64_t *__restrict__ x, int N, int V,
                                                   int D, int64_t ignore_index, int rows_per,
                                                   float *__restrict__ part,
                                                   int *__restrict__ cnt) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const int r0 = blockIdx.y * rows_per, r1 = min(N, r0 + rows_per);
  float acc = 0.0f;
  int c = 0;
  for (int n = r0; n < r1; ++n) {
    const int64_t xv = x[n];
    if (xv == ignore_index || xv < 0 || xv >= V) continue;
    ++c;
    if (d < D) acc += bf2f(E[(int64_t)n * D + d]);
  }
  if (d < D) part[(int64_t)blockIdx.y * D + d] = acc;
  if (blockIdx.x == 0 && threadIdx.x == 0) cnt[blockIdx.y] = c;
}

// mean row: fixed-order fp64 sums of the row-block partials / N_v (0 if none)
__global__ __launch_bounds__(256) void k_vo_mean(const float *__restrict__ part,
                                                 const int *__restrict__ cnt, int nrb, int D,
                                                 float *__restrict__ mean) {
  // nrb <= 256: one count per thread; integer sums are exact in any order
  __shared__ unsigned long long tot;
  if (threadIdx.x == 0) tot = 0ull;
  __syncthreads();
  if ((int)threadIdx.x < nrb) atomicAdd(&tot, (unsigned long long)cnt[threadIdx.x]);
  __syncthreads();
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  double s = 0.0;
#pragma unroll 8
  for (int i = 0; i < nrb; ++i) s += (double)part[(int64_t)i * D + d];
  mean[d] = tot > 0 ? (float)(s / (double)tot) : 0.0f;
}

// one wave per entry: the average logit and its sort key; entries past V
// (the padding to a power of two) get the largest key
__global__ __launch_bounds__(256) void k_vo_keys(const u16 *__restrict__ C,
                                                 const float *__restrict__ mean, int V, int D,
                                                 int P2, uint64_t *__restrict__ keys) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (v >= P2) return;
  if (v >= V) {
    if (l == 0) keys[v] = ~0ull;
    return;
  }
  float acc = 0.0f;
  for (int c = l; c < D / 8; c += 64) {
    const u32x4 q = *reinterpret_cast<const u32x4 *>(C + (int64_t)v * D + c * 8);
    const float *m = mean + c * 8;
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(__uint_as_float(w4[i] << 16), m[2 * i], acc);
      acc = fmaf(__uint_as_float(w4[i] & 0xffff0000u), m[2 * i + 1], acc);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (l == 0) {
    // ascending key = descending average; -0 as +0; NaN after every number
    uint32_t k;
    if (acc != acc) {
      k = 0xffffffffu;
    } else {
      const uint32_t u = acc == 0.0f ? 0u : __float_as_uint(acc);
      const uint32_t up = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // increasing in acc
      k = ~up;
    }
    keys[v] = ((uint64_t)k << 32) | (uint32_t)v;
  }
}

__device__ __forceinline__ void vo_cmpx(uint64_t &a, uint64_t &b, bool up) {
  if ((a > b) == up) {
    const uint64_t t = a;
    a = b;
    b = t;
  }
}

// Bitonic steps inside a 4096-key block in LDS.  full: every stage k = 2 ..
// min(4096, P2); else the steps j = 2048 .. 1 of stage k.  The pair (i, i + j)
// is sorted upwards when bit k of i is 0.
__global__ __launch_bounds__(VO_LTHREADS) void k_vo_sort_local(uint64_t *__restrict__ keys,
                                                               int P2, int k, int full) {
  __shared__ uint64_t sk[VO_LOCAL];
  const int n = min(P2, VO_LOCAL);
  const int base = blockIdx.x * n;
  for (int i = threadIdx.x; i < n; i += VO_LTHREADS) sk[i] = keys[base + i];
  __syncthreads();
  const int k0 = full ? 2 : k, k1 = full ? n : k;
  for (int kk = k0; kk <= k1; kk <<= 1) {
    for (int j = min(kk, n) >> 1; j >= 1; j >>= 1) {
      for (int p = threadIdx.x; p < n / 2; p += VO_LTHREADS) {
        const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));
        vo_cmpx(sk[i], sk[i + j], ((base + i) & kk) == 0);
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += VO_LTHREADS) keys[base + i] = sk[i];
}

// one bitonic step (k, j) with j >= 4096 over all keys, a pair per thread
__global__ __launch_bounds__(256) void k_vo_sort_global(uint64_t *__restrict__ keys, int P2,
                                                        int k, int j) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= P2 / 2) return;
  const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));
  uint64_t a = keys[i], b = keys[i + j];
  const bool up = (i & k) == 0;
  if ((a > b) == up) {
    keys[i] = b;
    keys[i + j] = a;
  }
}

__global__ __launch_bounds__(256) void k_vo_out(const uint64_t *__restrict__ keys, int V,
                                                int32_t *__restrict__ order) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < V) order[i] = (int32_t)(uint32_t)(keys[i] & 0xffffffffull);
}

// position of each entry in a vocabulary order: -1 everywhere, then the
// scatter (entries outside [0, V) are skipped)
__global__ __launch_bounds__(256) void k_vo_fill(int32_t *__restrict__ vpos, int V) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < V) vpos[i] = -1;
}
__global__ __launch_bounds__(256) void k_vo_pos(const int32_t *__restrict__ order, int V,
                                                int32_t *__restrict__ vpos) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= V) return;
  const int32_t g = order[i];
  if (g >= 0 && g < V) vpos[g] = i;
}

struct Plan {
  int64_t N, V, D;
  int64_t TT, VTf, S, Stot;       // forward: token tiles, full vocabulary tiles, slabs
                                  // over them, partials per token (+1 for a ragged tile)
  int64_t Npad, Dpad;             // backward padding
  int64_t Vc, nchunks, Vcpad;     // backward chunks
  int64_t Nb, ntb;                // backward token blocks: rows per block, blocks
  int64_t de_parts, de_kpart;     // dE split over each chunk's rows (1: no split)
  // forward workspace offsets
  size_t f_nv, f_pm, f_ps, f_tl, f_bs, f_perm, f_xc, f_ec, f_total;
  // backward workspace offsets
  size_t b_nv, b_cnt, b_slots, b_ri, b_srow, b_tl, b_et, b_ct, b_gnv, b_acc, b_flags, b_perm, b_xc, b_ec,
      b_vpos, b_dcacc, b_total;
  // vocabulary order (inside the backward workspace, used by its own call)
  int64_t P2, nrb, rows_per;
  size_t s_keys, s_part, s_cnt, s_mean;
  int64_t nslots;  // sigma, amax(E), amax(C)
};

// Compute units of the current device (the plans below fill whole rounds of
// them): 256 on an MI355X, and 256 when no device can be queried.
int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int n = 0;
    cache[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                      hipSuccess && n > 0) ? n : 256;
    (void)hipGetLastError();
  }
  return cache[dev];
}

Plan make_plan(int64_t N, int64_t V, int64_t D) {
  Plan p;
  const int64_t cus = device_cus();
  p.N = N;
  p.V = V;
  p.D = D;
  p.TT = cdiv(N, BN);
  p.VTf = V / BM;
  // Slabs over the full vocabulary tiles: the smallest multiple of 4 that
  // makes the workgroups (token tiles x slabs) a whole number of rounds on the
  // CUs (256), so every CU runs the same number of equally long slabs and none
  // idles at the end (at least 4, so the launch order's 4 x 8 tile groups
  // share each C tile among 8 workgroups and each E tile among 4); where that
  // takes more than 64 slabs, about 2048 workgroups.  A ragged last tile is
  // one more slab of its own (its own small launch).
  int64_t S = 1;
  if (p.TT > 0) {
    int64_t g = cus, t = p.TT % cus;
    while (t) { const int64_t r = g % t; g = t; t = r; }  // gcd(TT, cus)
    S = cus / g;
    if (S < 4) S = 4;
    if (S > 64) {
      S = cdiv(2048, p.TT);
      if (S >= 8) S &= ~(int64_t)7;
    }
  }
  if (S > p.VTf) S = p.VTf;
  if (S > 256) S = 256;
  p.S = S;  // 0 when V < 256: only the ragged slab
  p.Stot = S + ((V % BM) != 0 ? 1 : 0);
  p.Npad = rup(N, BM);
  p.Dpad = rup(D, BN);
  // Past TB_MAX rows the backward takes the tokens in blocks of at most
  // TB_ROWS (equal whole tiles): the G-hat buffers and unit maps are sized
  // for one block, dE keeps its accumulator over every row and dC gains one
  // over the chunk (Vcpad x Dpad fp32).  At 65,536 rows of width 2048 that
  // takes the G-hat double buffer from 2 GiB to 256 MiB.
  p.ntb = p.Npad > TB_MAX ? cdiv(p.Npad, TB_ROWS) : 1;
  p.Nb = p.ntb > 1 ? rup(cdiv(p.Npad, p.ntb), BN) : p.Npad;
  // Few dE tiles against the CUs (256): each tile is dealt over parts of the
  // chunk's rows, 64-row steps each, so no dE tile outlasts the rest of its
  // launch; the parts of the first (longest) chunk are the most any chunk
  // has.  Each part reads and writes its own accumulator per chunk, so the
  // split pays only while the dE tiles are the launch's longest path:
  // under 48 tiles up to 8 parts (36 tiles: 13% faster eight ways), up to 96
  // tiles two (64 tiles, the Qwen2.5-0.5B head shape: backward 7% faster two
  // ways, 2% slower four ways).
  const int64_t nEt = (p.Npad / BM) * (p.Dpad / BN);
  int64_t parts = 1;
  if (p.ntb > 1) parts = 1;  // token blocks: no split
  else if (nEt > 0 && nEt < cus * 3 / 16) parts = std::min<int64_t>(8, cdiv(cus, nEt));
  else if (nEt > 0 && nEt <= cus * 3 / 8) parts = 2;
  const int64_t vchunk = vchunk_for(p.Npad, p.Dpad, parts);
  p.Vc = V < vchunk ? rup(V, BM) : vchunk;
  p.nchunks = cdiv(V, p.Vc);
  p.Vcpad = rup(V < vchunk ? V : vchunk, BM);

  size_t o = 0;
  p.f_nv = o; o = align256(o + 8);
  p.f_pm = o; o = align256(o + (size_t)(p.Stot * N) * 4);
  p.f_ps = o; o = align256(o + (size_t)(p.Stot * N) * 4);
  p.f_tl = o; o = align256(o + (size_t)N * 8);
  p.f_bs = o; o = align256(o + (size_t)cdiv(N, 256) * 8);
  // the compacted rows: order, targets, E rows
  p.f_perm = o; o = align256(o + (size_t)N * 4);
  p.f_xc = o; o = align256(o + (size_t)N * 8);
  p.f_ec = o; o = align256(o + (size_t)(N * D) * 2);
  p.f_total = o;

  o = 0;
  p.b_nv = o; o = align256(o + 8);
  p.b_cnt = o; o = align256(o + (size_t)NCOUNT * 8);
  p.nslots = 3;
  p.b_slots = o; o = align256(o + (size_t)p.nslots * 4);
  p.b_ri = o; o = align256(o + (size_t)p.Npad * sizeof(RowInfo));
  p.b_srow = o; o = align256(o + (size_t)p.Npad * 4);
  p.b_tl = o; o = align256(o + (size_t)N * 8);
  p.b_et = o; o = align256(o + (size_t)(p.Dpad * p.Npad) * 2);
  // chunk buffers come in pairs: chunk c uses copy c & 1
  p.b_ct = o; o = align256(o + 2 * (size_t)(p.Dpad * p.Vcpad) * 2);
  p.b_gnv = o; o = align256(o + 2 * (size_t)(p.Nb * p.Vcpad) * 2);
  // dE accumulator: one 256 x 256 fp32 block per dE tile, in register order
  p.de_kpart = rup(cdiv(p.Vcpad, parts), 64);
  p.de_parts = cdiv(p.Vcpad, p.de_kpart);
  const bool split = p.de_parts > 1;
  p.b_acc = o;
  o = align256(o + (p.nchunks > 1 || split ? (size_t)(p.de_parts * p.Npad * p.Dpad) * 4 : 0));
  p.b_flags = o; o = align256(o + 4 * (size_t)(p.Vcpad / UNIT) * (size_t)(p.Nb / UNIT));
  p.b_perm = o; o = align256(o + (size_t)p.Npad * 4);  // read 4 rows at a time
  p.b_xc = o; o = align256(o + (size_t)N * 8);
  p.b_ec = o; o = align256(o + (size_t)(N * D) * 2);
  p.b_vpos = o; o = align256(o + (size_t)V * 4);  // sorted backward: position of each entry
  p.b_dcacc = o; o = align256(o + (p.ntb > 1 ? (size_t)(p.Vcpad * p.Dpad) * 4 : 0));
  p.b_total = o;

  // vocabulary order: the sort keys padded to a power of two (at least one
  // LDS block), the mean row's partial sums over at most VO_RB row blocks
  p.P2 = VO_LOCAL;
  while (p.P2 < V) p.P2 <<= 1;
  p.nrb = N > 0 ? std::min<int64_t>(cdiv(N, 64), VO_RB) : 1;
  p.rows_per = N > 0 ? cdiv(N, p.nrb) : 0;
  if (N > 0) p.nrb = cdiv(N, p.rows_per);
  o = 0;
  p.s_keys = o; o = align256(o + (size_t)p.P2 * 8);
  p.s_part = o; o = align256(o + (size_t)(p.nrb * D) * 4);
  p.s_cnt = o; o = align256(o + (size_t)p.nrb * 4);
  p.s_mean = o; o = align256(o + (size_t)D * 4);
  if (o > p.b_total) p.b_total = o;
  return p;
}

bool shape_ok(int64_t N, int64_t V, int64_t D) {
  if (N < 0 || V < 1 || D < 8 || (D % 8) != 0) return false;
  // index arithmetic limits: 32-bit tile offsets and counts
  if (N > (int64_t)1 << 21 || V > (int64_t)1 << 30 || D > 16384) return false;
  if ((int64_t)BM * D * 2 >= ((int64_t)1 << 31)) return false;
  return true;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---- profiling --------------------------------------------------------------
struct ProfRec {
  const char *name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof = false;
// cce_profile_enable(2): each role of a backward step in a launch of its own
bool g_prof_roles = false;
std::vector<ProfRec> g_recs;

void prof_clear() {
  for (auto &r : g_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
}

struct ProfScope {
  const char *name;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(const char *n, hipStream_t s) : name(n), st(s) {
    // timing only, read after the stream is synchronised: no system-scope
    // fence (a cache write-back and invalidation at each record)
    if (g_prof && hipEventCreateWithFlags(&a, hipEventDisableSystemFence) == hipSuccess &&
        hipEventCreateWithFlags(&b, hipEventDisableSystemFence) == hipSuccess)
      (void)hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (a && b) {
      (void)hipEventRecord(b, st);
      std::lock_guard<std::mutex> g(g_prof_mu);
      g_recs.push_back({name, a, b});
    }
  }
};

#define LAUNCH(NAME, STREAM, ...)                                    \
  do {                                                               \
    ProfScope _ps(NAME, STREAM);                                     \
    __VA_ARGS__;                                                     \
    if (hipGetLastError() != hipSuccess) return CCE_ERR_HIP;        \
  } while (0)

}  // namespace

namespace {

cce_status forward_impl(const void *E, const void *C, const int64_t *x, int64_t N, int64_t V,
                        int64_t D, int64_t ignore_index, int reduction, float *loss, float *lse,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (!shape_ok(N, V, D)) return CCE_ERR_BAD_SHAPE;
  if (reduction < CCE_REDUCTION_NONE || reduction > CCE_REDUCTION_SUM) return CCE_ERR_BAD_REDUCTION;
  if (!C || !workspace || !loss) return CCE_ERR_NULL_POINTER;
  if (N > 0 && (!E || !x || !lse)) return CCE_ERR_NULL_POINTER;
  if (!aligned(C, 16) || !aligned(workspace, 16) || (E && !aligned(E, 16)) ||
      (x && !aligned(x, 8)) || !aligned(loss, 4) || (lse && !aligned(lse, 4)))
    return CCE_ERR_BAD_ALIGNMENT;
  const Plan p = make_plan(N, V, D);
  if (workspace_bytes < p.f_total) return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  int64_t *nv = (int64_t *)(ws + p.f_nv);
  float *pm = (float *)(ws + p.f_pm);
  float *ps = (float *)(ws + p.f_ps);
  double *tl = (double *)(ws + p.f_tl);
  double *bs = (double *)(ws + p.f_bs);
  int32_t *perm = (int32_t *)(ws + p.f_perm);
  int64_t *xc = (int64_t *)(ws + p.f_xc);
  u16 *Ec = (u16 *)(ws + p.f_ec);
  const u16 *Ch = (const u16 *)C;

  // ignored rows to the end; from here on every kernel sees the compacted
  // rows (Ec, xc) and stops at the valid count
  LAUNCH("small", st,
         k_compact<<<1, 1024, 0, st>>>(x, (int)N, ignore_index, perm, xc, nv, nullptr, nullptr, 0));
  if (N > 0) {
    LAUNCH("gather", st,
           k_gather_rows<<<(int)std::min<int64_t>(cdiv(N * D / 8, 256), 4096), 256, 0, st>>>(
               (const u16 *)E, perm, (int)N, (int)D, nv, Ec));
    const u16 *Eh = Ec;
    // the target logits (the merge adds them to the other entries' partials)
    LAUNCH("target", st,
           k_target<<<(int)cdiv(N, 4), 256, 0, st>>>(Ch, Eh, xc, (int)N, (int)V, (int)D,
                                                     ignore_index, tl));
    // the S slabs of full tiles; a ragged last tile is slab S, alone in a
    // launch of its own that masks its rows past V
    if (p.S > 0)
      LAUNCH("fwd_lse", st,
             k_fwd_lse<false><<<(int)(p.TT * p.S), NTHREADS, 0, st>>>(
                 Ch, Eh, (int)N, (int)V, (int)D, (int)p.TT, (int)p.VTf, 0, 0, (int)p.S, xc,
                 ignore_index, pm, ps, nv));
    if (p.Stot > p.S)
      LAUNCH("fwd_lse", st,
             k_fwd_lse<true><<<(int)p.TT, NTHREADS, 0, st>>>(Ch, Eh, (int)N, (int)V, (int)D,
                                                              (int)p.TT, 1, (int)p.VTf, (int)p.S,
                                                              1, xc, ignore_index, pm, ps,
                                                              nv));
    LAUNCH("fwd_merge", st,
           k_fwd_merge<<<(int)cdiv(N, 256), 256, 0, st>>>(pm, ps, tl, xc, perm, (int)N, (int)V,
                                                          (int)p.Stot, ignore_index, reduction,
                                                          loss, lse, bs));
  }
  if (reduction != CCE_REDUCTION_NONE)
    LAUNCH("small", st,
           k_fwd_reduce<<<1, 256, 0, st>>>(bs, (int)cdiv(N, 256), nv, reduction, loss));
  return CCE_OK;
}

// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the forward's workspace in
// a static device array.  Each GPU the library runs on holds its own copy
// until the process ends; in host code the array's name is only a stand-in,
// so its device address is taken once per device with hipGetSymbolAddress
// and that address is what the kernels receive.  Every call on a GPU shares
// its copy: calls that overlap on one GPU race.
static __device__ __align__(256) unsigned char scratch[CCE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

// the calling thread's current device's copy of `scratch`
cce_status scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return CCE_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CCE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CCE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char *cce_status_string(cce_status s) {
  switch (s) {
    case CCE_OK: return "ok";
    case CCE_ERR_NULL_POINTER: return "null pointer argument";
    case CCE_ERR_BAD_SHAPE: return "bad shape (need N >= 0, V >= 1, D >= 8, D % 8 == 0, within limits)";
    case CCE_ERR_BAD_REDUCTION: return "bad reduction";
    case CCE_ERR_BAD_ALIGNMENT: return "misaligned pointer (16 bytes for E, C, dE, dC, workspace)";
    case CCE_ERR_BAD_EPS: return "filter_eps must be finite and >= 0";
    case CCE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than cce_workspace_bytes";
    case CCE_ERR_HIP: return "HIP launch error";
    case CCE_ERR_BAD_FILTER_MODE: return "filter_mode must be CCE_FILTER_BOTH, _FULL_C or _FULL_E";
    case CCE_ERR_SCRATCH_TOO_SMALL:
      return "the forward's workspace at this shape exceeds CCE_NOALLOC_SCRATCH_BYTES";
  }
  return "unknown status";
}

cce_status cce_workspace_bytes(int64_t N, int64_t V, int64_t D, size_t *fwd_bytes,
                               size_t *bwd_bytes) {
  if (!shape_ok(N, V, D)) return CCE_ERR_BAD_SHAPE;
  const Plan p = make_plan(N, V, D);
  if (fwd_bytes) *fwd_bytes = p.f_total;
  if (bwd_bytes) *bwd_bytes = p.b_total;
  return CCE_OK;
}

cce_status cce_forward(const void *E, const void *C, const int64_t *x, int64_t N, int64_t V,
                       int64_t D, int64_t ignore_index, int reduction, float *loss, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(E, C, x, N, V, D, ignore_index, reduction, loss, lse, workspace,
                      workspace_bytes, stream);
}

cce_status cce_forward_noalloc(const void *E, const void *C, const int64_t *x, int64_t N,
                               int64_t V, int64_t D, int64_t ignore_index, int reduction,
                               float *loss, float *lse, void *stream) {
  if (!shape_ok(N, V, D)) return CCE_ERR_BAD_SHAPE;
  if (make_plan(N, V, D).f_total > (size_t)CCE_NOALLOC_SCRATCH_BYTES) return CCE_ERR_SCRATCH_TOO_SMALL;
  void *ws = nullptr;
  const cce_status rc = scratch_address(&ws);
  if (rc != CCE_OK) return rc;
  return forward_impl(E, C, x, N, V, D, ignore_index, reduction, loss, lse, ws,
                      (size_t)CCE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {
// The backward; vorder (nullable) is a vocabulary order: chunk rows, filter
// units and targets follow it, dC rows go back to their entries.
cce_status backward_impl(const void *E, const void *C, const int64_t *x, const float *lse,
                         const float *grad_loss, int64_t N, int64_t V, int64_t D,
                         int64_t ignore_index, int reduction, float filter_eps, int filter_mode,
                         const int32_t *vorder, void *dE, void *dC, cce_filter_stats *stats,
                         void *workspace, size_t workspace_bytes, void *stream) {
  if (!shape_ok(N, V, D)) return CCE_ERR_BAD_SHAPE;
  if (reduction < CCE_REDUCTION_NONE || reduction > CCE_REDUCTION_SUM) return CCE_ERR_BAD_REDUCTION;
  if (!(filter_eps >= 0.0f) || !isfinite(filter_eps)) return CCE_ERR_BAD_EPS;
  if (filter_mode != CCE_FILTER_BOTH && filter_mode != CCE_FILTER_FULL_C &&
      filter_mode != CCE_FILTER_FULL_E)
    return CCE_ERR_BAD_FILTER_MODE;
  if (!C || !dC || !workspace) return CCE_ERR_NULL_POINTER;
  if (N > 0 && (!E || !x || !lse || !grad_loss || !dE)) return CCE_ERR_NULL_POINTER;
  if (!aligned(C, 16) || !aligned(dC, 16) || !aligned(workspace, 16) ||
      (E && !aligned(E, 16)) || (dE && !aligned(dE, 16)) || (x && !aligned(x, 8)) ||
      (lse && !aligned(lse, 4)) || (grad_loss && !aligned(grad_loss, 4)) ||
      (stats && !aligned(stats, 8)))
    return CCE_ERR_BAD_ALIGNMENT;
  const Plan p = make_plan(N, V, D);
  if (workspace_bytes < p.b_total) return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  int64_t *nv = (int64_t *)(ws + p.b_nv);
  unsigned long long *cnt = (unsigned long long *)(ws + p.b_cnt);
  RowInfo *ri = (RowInfo *)(ws + p.b_ri);
  float *srow = (float *)(ws + p.b_srow);
  double *tl = (double *)(ws + p.b_tl);
  u16 *Et = (u16 *)(ws + p.b_et);
  u16 *Ct = (u16 *)(ws + p.b_ct);
  u16 *Gnv = (u16 *)(ws + p.b_gnv);
  float *acc = (float *)(ws + p.b_acc);
  uint32_t *slots = (uint32_t *)(ws + p.b_slots);
  uint32_t *sigma = slots, *amaxE = slots + 1, *amaxC = slots + 2;
  // per copy: the C operand, G-hat and each unit map (G-hat and the maps for one token block)
  const size_t ct_elems = (size_t)(p.Dpad * p.Vcpad), g_elems = (size_t)(p.Vcpad * p.Nb);
  const size_t map_bytes = (size_t)(p.Vcpad / UNIT) * (size_t)(p.Nb / UNIT);
  uint8_t *maps = (uint8_t *)(ws + p.b_flags);  // [copy][map2, map3]
  int32_t *perm = (int32_t *)(ws + p.b_perm);
  int64_t *xc = (int64_t *)(ws + p.b_xc);
  u16 *Ec = (u16 *)(ws + p.b_ec);
  int32_t *vpos = vorder ? (int32_t *)(ws + p.b_vpos) : nullptr;
  const u16 *Eh = Ec;  // the compacted rows (gathered below)
  const u16 *Ch = (const u16 *)C;
  const int Npad = (int)p.Npad, Dpad = (int)p.Dpad;
  const int DT = (int)(p.Dpad / BN);
  const float eps = filter_eps;
  // the threshold of each contraction's G-hat (0: every unit kept)
  const float eps_dE = filter_mode == CCE_FILTER_FULL_E ? 0.0f : eps;
  const float eps_dC = filter_mode == CCE_FILTER_FULL_C ? 0.0f : eps;

  // ignored rows to the end (as in the forward); every kernel below works on
  // the compacted rows and stops at the valid count
  LAUNCH("small", st,
         k_compact<<<1, 1024, 0, st>>>(x, (int)N, ignore_index, perm, xc, nv, cnt, slots,
                                       (int)p.nslots));
  if (N > 0) {
    LAUNCH("gather", st,
           k_gather_rows<<<(int)std::min<int64_t>(cdiv(N * D / 8, 256), 4096), 256, 0, st>>>(
               (const u16 *)E, perm, (int)N, (int)D, nv, Ec));
    if (vorder) {
      LAUNCH("small", st, k_vo_fill<<<(int)cdiv(V, 256), 256, 0, st>>>(vpos, (int)V));
      LAUNCH("small", st, k_vo_pos<<<(int)cdiv(V, 256), 256, 0, st>>>(vorder, (int)V, vpos));
    }
    LAUNCH("target", st,
           k_target<<<(int)cdiv(N, 4), 256, 0, st>>>(Ch, Eh, xc, (int)N, (int)V, (int)D,
                                                     ignore_index, tl));
    LAUNCH("small", st,
           k_bwd_rows<<<(int)cdiv(Npad, 256), 256, 0, st>>>(xc, perm, lse, grad_loss, (int)N,
                                                            Npad, (int)V, (int)D, ignore_index,
                                                            reduction, nv, tl, ri, srow, sigma,
                                                            (u16 *)dE, vpos));
    const int64_t c8 = N * D / 8;
    LAUNCH("transpose", st,
           k_amax<<<(int)(cdiv(c8, 256) < 256 ? cdiv(c8, 256) : 256), 256, 0, st>>>(Eh, c8,
                                                                                     amaxE));
    LAUNCH("transpose", st,
           k_transpose<<<dim3(Npad / 64, Dpad / 64), 256, 0, st>>>(Eh, (int)N, (int)D, (int)D, Et,
                                                                  amaxE, srow, sigma));
    // one power-of-two scale for every C chunk (the chunks' transposes run
    // inside the backward launches)
    const int64_t cc8 = V * D / 8;
    LAUNCH("transpose", st,
           k_amax<<<(int)(cdiv(cc8, 256) < 4096 ? cdiv(cc8, 256) : 4096), 256, 0, st>>>(Ch, cc8,
                                                                                       amaxC));
  }
  // The backward walks (chunk, token block) pairs, the blocks inside each
  // chunk (one block of every row unless the plan blocks the tokens).
  // Launch j runs the dC / dE tiles of pair j - 1, then the G-hat tiles of
  // pair j and, at a chunk's first block, the dE operand (scaled fp16
  // transpose) of its C rows (absent past the last pair or when N == 0).
  // G-hat and the unit maps alternate between two copies by pair, the C
  // operand by chunk.
  const int64_t ntb = p.ntb, npairs = p.nchunks * ntb;
  const int Nb = (int)p.Nb;
  float *dcacc = ntb > 1 ? (float *)(ws + p.b_dcacc) : nullptr;
  for (int64_t j = 0; j <= npairs; ++j) {
    DcArgs dca{};
    DeArgs dea{};
    GradArgs gra{};
    int nC = 0, nE = 0, nG = 0;
    if (j >= 1) {
      const int64_t q = j - 1, c = q / ntb, tb = q % ntb;
      const int gb = (int)(q & 1), cb = (int)(c & 1);
      const int r0 = (int)(tb * Nb), rows = (int)std::min<int64_t>(Nb, Npad - r0);
      const int v_start = (int)(c * p.Vc);
      const int chunk_len = (int)((V - v_start) < p.Vc ? (V - v_start) : p.Vc);
      const int cpad = (int)rup(chunk_len, BM);
      u16 *Ctb = Ct + cb * ct_elems;
      uint8_t *m2 = maps + (size_t)gb * 2 * map_bytes;
      const int dmode = ntb == 1 ? 3 : (tb == 0 ? 1 : 0) | (tb == ntb - 1 ? 2 : 0);
      dca = DcArgs{Gnv + gb * g_elems, Nb, Et + (size_t)r0 * Dpad, rows, chunk_len, v_start,
                   (int)D, DT, cpad / BM, (u16 *)dC, sigma, amaxE, m2, Nb / UNIT, nv,
                   eps_dC > 0.0f ? 1 : 0, vorder, (int)V, r0, dcacc, dmode};
      nC = (cpad / BM) * DT;
      if (N > 0) {
        // split: every chunk, the last included, leaves its sums in the
        // parts' accumulators (k_de_final casts them)
        const bool split = p.de_parts > 1;
        const int mode = (c == 0 ? 1 : 0) | (c == p.nchunks - 1 && !split ? 2 : 0);
        const int kpart = split ? (int)p.de_kpart : cpad;
        dea = DeArgs{Gnv + gb * g_elems, Nb, Ctb, cpad, (int)std::min<int64_t>(rows, N - r0),
                     (int)D, DT, rows / BM, mode, acc + (size_t)r0 * Dpad, (u16 *)dE,
                     srow + r0, amaxC, m2 + map_bytes, cpad / UNIT, nv, perm + r0,
                     eps_dE > 0.0f ? 1 : 0, kpart, (int)cdiv(cpad, kpart),
                     (int64_t)Npad * Dpad, r0};
        nE = (rows / BM) * DT;
      }
    }
    TrArgs tra{};
    int nT = 0;
    if (j < npairs && N > 0) {
      const int64_t c = j / ntb, tb = j % ntb;
      const int gb = (int)(j & 1), cb = (int)(c & 1);
      const int r0 = (int)(tb * Nb), rows = (int)std::min<int64_t>(Nb, Npad - r0);
      const int v_start = (int)(c * p.Vc);
      const int chunk_len = (int)((V - v_start) < p.Vc ? (V - v_start) : p.Vc);
      const int cpad = (int)rup(chunk_len, BM);
      uint8_t *m2 = maps + (size_t)gb * 2 * map_bytes;
      gra = GradArgs{Ch, Eh + (size_t)r0 * D, ri + r0, (int)std::min<int64_t>(rows, N - r0),
                     (int)V, (int)D, v_start, chunk_len, rows / BN, cpad / BM, eps_dE, eps_dC,
                     Gnv + gb * g_elems, Nb, cnt, m2, m2 + map_bytes, Nb / UNIT, cpad / UNIT,
                     nv, vorder, r0};
      nG = (cpad / BM) * (rows / BN);
      if (tb == 0) {
        // the C chunk's operand for dE, used by the chunk's dE launches
        tra = TrArgs{Ch, chunk_len, (int)D, v_start, Ct + cb * ct_elems, DT, amaxC, vorder,
                     (int)V};
        nT = (cpad / BM) * DT;
      }
    }
    const int nCp = (int)rup(nC, 8), nEp = (int)rup((int64_t)nE * (nE ? dea.nparts : 1), 8);
    // the contraction whose K is longer goes first: dC sums over the tokens,
    // dE over the chunk (or its part)
    const int dcf = (nE && dca.Kn > dea.kpart) ? 1 : 0;
    const int nGp = (int)rup(nG, 8);
    if (nCp + nEp + nGp + nT > 0) {
      const int nb = nCp + nEp + nGp + nT;
      if (vorder)
        LAUNCH("bwd_step", st,
               k_bwd_step<true><<<nb, NTHREADS, 0, st>>>(dca, nC, nCp, dea, nE, nEp, gra, nG, nGp,
                                                         tra, nT, dcf, nv));
      else if (g_prof_roles) {
        // the same tiles, one role per launch, in the fused launch's order
        // (the roles of a launch touch disjoint buffers)
        if (nEp)
          LAUNCH("bwd_de", st, k_bwd_step<false><<<nEp, NTHREADS, 0, st>>>(
                                   dca, 0, 0, dea, nE, nEp, gra, 0, 0, tra, 0, 0, nv));
        if (nCp)
          LAUNCH("bwd_dc", st, k_bwd_step<false><<<nCp, NTHREADS, 0, st>>>(
                                   dca, nC, nCp, dea, 0, 0, gra, 0, 0, tra, 0, 0, nv));
        if (nGp)
          LAUNCH("bwd_g", st, k_bwd_step<false><<<nGp, NTHREADS, 0, st>>>(
                                  dca, 0, 0, dea, 0, 0, gra, nG, nGp, tra, 0, 0, nv));
        if (nT)
          LAUNCH("bwd_t", st, k_bwd_step<false><<<nT, NTHREADS, 0, st>>>(
                                  dca, 0, 0, dea, 0, 0, gra, 0, 0, tra, nT, 0, nv));
      } else
        LAUNCH("bwd_step", st,
               k_bwd_step<false><<<nb, NTHREADS, 0, st>>>(dca, nC, nCp, dea, nE, nEp, gra, nG,
                                                          nGp, tra, nT, dcf, nv));
    }
  }
  if (N > 0 && p.de_parts > 1) {
    const int nE = (int)((p.Npad / BM) * (p.Dpad / BN));
    LAUNCH("small", st,
           k_de_final<<<(int)((int64_t)nE * NWAVES * MB * NB * 64 / 256), 256, 0, st>>>(
               acc, (int64_t)Npad * Dpad, (int)p.de_parts, nE, Npad / BM, DT, (int)D, nv, perm,
               (u16 *)dE));
  }
  if (stats) LAUNCH("small", st, k_stats<<<1, 64, 0, st>>>(cnt, nv, V, eps > 0.0f ? 1 : 0, stats));
  return CCE_OK;
}
}  // namespace

extern "C" {

cce_status cce_backward_ex(const void *E, const void *C, const int64_t *x, const float *lse,
                           const float *grad_loss, int64_t N, int64_t V, int64_t D,
                           int64_t ignore_index, int reduction, float filter_eps,
                           int filter_mode, void *dE, void *dC, cce_filter_stats *stats,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return backward_impl(E, C, x, lse, grad_loss, N, V, D, ignore_index, reduction, filter_eps,
                       filter_mode, nullptr, dE, dC, stats, workspace, workspace_bytes, stream);
}

cce_status cce_backward_sorted(const void *E, const void *C, const int64_t *x, const float *lse,
                               const float *grad_loss, int64_t N, int64_t V, int64_t D,
                               int64_t ignore_index, int reduction, float filter_eps,
                               int filter_mode, const int32_t *vocab_order, void *dE, void *dC,
                               cce_filter_stats *stats, void *workspace, size_t workspace_bytes,
                               void *stream) {
  if (!shape_ok(N, V, D)) return CCE_ERR_BAD_SHAPE;
  // gathered C rows are addressed by 32-bit buffer offsets
  if (V * D * 2 > (int64_t)OOB) return CCE_ERR_BAD_SHAPE;
  if (!vocab_order) return CCE_ERR_NULL_POINTER;
  if (!aligned(vocab_order, 4)) return CCE_ERR_BAD_ALIGNMENT;
  return backward_impl(E, C, x, lse, grad_loss, N, V, D, ignore_index, reduction, filter_eps,
                       filter_mode, vocab_order, dE, dC, stats, workspace, workspace_bytes,
                       stream);
}

cce_status cce_vocab_order(const void *E, const void *C, const int64_t *x, int64_t N, int64_t V,
                           int64_t D, int64_t ignore_index, int32_t *order, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (!shape_ok(N, V, D)) return CCE_ERR_BAD_SHAPE;
  if (!C || !order || !workspace) return CCE_ERR_NULL_POINTER;
  if (N > 0 && (!E || !x)) return CCE_ERR_NULL_POINTER;
  if (!aligned(C, 16) || !aligned(order, 4) || !aligned(workspace, 16) ||
      (E && !aligned(E, 16)) || (x && !aligned(x, 8)))
    return CCE_ERR_BAD_ALIGNMENT;
  const Plan p = make_plan(N, V, D);
  if (workspace_bytes < p.b_total) return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  uint64_t *keys = (uint64_t *)(ws + p.s_keys);
  float *part = (float *)(ws + p.s_part);
  int *cnt = (int *)(ws + p.s_cnt);
  float *mean = (float *)(ws + p.s_mean);
  const int P2 = (int)p.P2, nrb = (int)p.nrb;
  const int dblocks = (int)cdiv(D, 256);
  LAUNCH("vocab_order", st,
         k_vo_rowsum<<<dim3(dblocks, nrb), 256, 0, st>>>((const u16 *)E, x, (int)N, (int)V,
                                                         (int)D, ignore_index, (int)p.rows_per,
                                                         part, cnt));
  LAUNCH("vocab_order", st, k_vo_mean<<<dblocks, 256, 0, st>>>(part, cnt, nrb, (int)D, mean));
  LAUNCH("vocab_order", st,
         k_vo_keys<<<P2 / 4, 256, 0, st>>>((const u16 *)C, mean, (int)V, (int)D, P2, keys));
  LAUNCH("vocab_order", st, k_vo_sort_local<<<P2 / VO_LOCAL, VO_LTHREADS, 0, st>>>(keys, P2, 0, 1));
  for (int k = 2 * VO_LOCAL; k <= P2; k <<= 1) {
    for (int j = k / 2; j >= VO_LOCAL; j >>= 1)
      LAUNCH("vocab_order", st,
             k_vo_sort_global<<<(int)cdiv(P2 / 2, 256), 256, 0, st>>>(keys, P2, k, j));
    LAUNCH("vocab_order", st, k_vo_sort_local<<<P2 / VO_LOCAL, VO_LTHREADS, 0, st>>>(keys, P2, k, 0));
  }
  LAUNCH("vocab_order", st, k_vo_out<<<(int)cdiv(V, 256), 256, 0, st>>>(keys, (int)V, order));
  return CCE_OK;
}

cce_status cce_backward(const void *E, const void *C, const int64_t *x, const float *lse,
                        const float *grad_loss, int64_t N, int64_t V, int64_t D,
                        int64_t ignore_index, int reduction, float filter_eps, void *dE, void *dC,
                        cce_filter_stats *stats, void *workspace, size_t workspace_bytes,
                        void *stream) {
  return cce_backward_ex(E, C, x, lse, grad_loss, N, V, D, ignore_index, reduction, filter_eps,
                         CCE_FILTER_BOTH, dE, dC, stats, workspace, workspace_bytes, stream);
}

cce_status cce_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (on < 0 || on > 2) return CCE_ERR_BAD_SHAPE;
  prof_clear();
  g_prof = on != 0;
  g_prof_roles = on == 2;
  return CCE_OK;
}

cce_status cce_profile_query(const char *name, int64_t *launches, double *total_ms) {
  if (!name || !launches || !total_ms) return CCE_ERR_NULL_POINTER;
  std::lock_guard<std::mutex> g(g_prof_mu);
  int64_t n = 0;
  double tot = 0.0;
  for (auto &r : g_recs) {
    if (strcmp(r.name, name) != 0) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return CCE_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return CCE_ERR_HIP;
    ++n;
    tot += ms;
  }
  *launches = n;
  *total_ms = tot;
  return CCE_OK;
}

}  // extern "C"
