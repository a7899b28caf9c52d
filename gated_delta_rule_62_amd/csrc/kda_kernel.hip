// Fused KDA recurrent prefill forward for gfx950 (CDNA4).
//
// The same kernel template also runs the two halves of the two-kernel split
// (FlashKDA's prep and recurrent kernels as the FlashInfer PR #4262 summary
// describes them): a token-parallel kernel that prepares one chunk of one head per
// workgroup and stores what the state side reads as a workspace record, and a
// recurrent kernel that copies the records back into LDS instead of preparing the
// chunks.  Both run this file's own preparation and state-side code, so the split
// gives the fused kernel's results bit for bit.
//
// One workgroup owns one (sequence n, head h, value tile j) work item and walks
// that sequence's chunks in order.  The fp32 state stays in MFMA accumulator
// registers for the whole sequence (the FlashInfer PR #4262 summary keeps it
// resident too, section 6, in tensor memory; here it is the accumulator file).
//
// Per chunk of C tokens (FlashInfer PR #4262 summary, sections 1-3):
//   1. load q, k, g, v, beta; L2-normalise q and k;
//      gate lam2 = lb*log2(e)*sigmoid(exp(A_log)*(g + dt_bias)) (base 2)
//   2. inclusive prefix G over the chunk per key column; a = 2^G_T
//   3. operands (bf16, round to nearest even):
//        centred  Qc = qh 2^(G-Ca), Kc = kh 2^(G-Ca), Ki = kh 2^(Ca-G)
//        decayed  Kr = kh 2^(G_T-G)
//      with a fixed anchor Ca (section 2 centres 32-token chunks on 16 b; any
//      anchor gives the same products, see below)
//   4. L = strictLower(diag(beta) Kc Ki^T), Mqk = lowerTri(Qc Ki^T)  (bf16 MFMA,
//      masked by select so overflowed upper entries never propagate)
//   5. (I + L)^-1 in fp32 on the 16x16 diagonal blocks (forward substitution);
//      the lower-left block is applied as a blocked solve in step 6
//   6. state side, per wave on its own value columns (section 3):
//        P^T = Kd S^T, O0 = S Qd^T, R^T = diag(beta)(V - P^T), U^T = (I+L)^-1 R^T,
//        S^T <- diag(a) S^T + Kr^T U^T,  O = O0 + U Mqk^T
//      where the decayed operands Qd = qh 2^G = 2^Ca Qc and Kd = 2^Ca Kc are
//      never formed: P^T = 2^Ca (Kc S^T) and O = 2^Ca (S Qc^T + U (2^-Ca Mqk)^T),
//      the power of two applied to the fp32 results.
//
// Anchor.  The prefix of a chunk of C tokens lies in [C b, 0] (b = lb log2(e)); the
// anchor is its middle, Ca = C b / 2 (section 2's 16 b for 32-token chunks), so the centred
// operands span 2^(Ca) .. 2^(-Ca) times a component of qh or kh, at most 2^118
// for the spans the host admits, with as much room above the bf16 normal minimum
// as below its maximum.  The state side runs 2^16 below scale: the accumulators
// hold S 2^-16 and the solve yields U 2^-16 (power-of-two factors folded into
// the solve operands, exact), so the unscaled products S Qc^T and S Kc^T stay
// inside fp32 for state rows up to 2^25 in 1-norm; 2^(Ca + 16) restores P and
// O, and the state is rescaled once on load and store.  The output scale is
// applied with that factor rather than folded into qh.
//
// Short chunks.  A chunk may hold fewer tokens than the tile has rows (8, 4, 2 or
// 1 in a 16-row tile): the empty rows are handled exactly like a ragged tail (zero
// inputs, no decay, beta 0, no stores), and the decay span, hence the anchor, is
// that of the tokens the chunk holds.  This admits strongly negative lower bounds
// whose 16-token span would leave the bf16 window.  Past |lb| log2(e) = 236 even one
// token's decay can leave it; one-token chunks then floor the per-token base-2 decay
// at -236, a factor below 1e-71, which changes no result representable in fp32.
//
// Schedule.  Steps 1-5 only touch chunk-local data, step 6 is the strictly
// ordered recurrence (section 3's scheduling property).  The state waves hold the
// state; the others (job waves) run chunk-local work.  Step s of the main loop has
// two phases separated by workgroup barriers that fence LDS only, so raw inputs
// loaded into registers a step ahead stay in flight.  Two LDS slots hold the
// prepared operands of chunks s and s+1 (the page's prep ring, two deep here).
// Two schedules:
//   state-only (twelve waves: four state waves, eight job waves; value tile D):
//   A  four matrix tiles of chunk s, P^T, O0 and the decay of S, R^T (state waves)
//      | q, k, v loads of s+2; norms, operands and value tile of s+1 (job waves)
//   B  blocked solve, output and state update of chunk s (state waves)
//      | the two inverted diagonal tiles of s+1 (job waves 4, 5); g loads of s+3,
//        gate and prefix of s+2 (job waves 0-3)
//   role split (eight waves: four state waves, four job waves):
//   A  P^T, O0 and the decay of S, then gate and prefix of s+1, then R^T (state
//      waves) | L, Mqk and the diagonal inverse blocks of chunk s, value tile of
//      s+1 (job waves)
//   B  blocked solve, state update and output of chunk s (state waves) | norms
//      and exponent-scaled operands of s+1 (every wave)
// An opt-in mode keeps the state in LDS as bf16 instead (FlashKDA's storage, the
// page on its bf16 state): the state-only schedule with the state widened, decayed,
// updated in fp32 and rounded back once per chunk.
//
// Layout of the state in registers.  Each wave holds S^T (K rows x its value
// columns) as 16x16 fp32 accumulator tiles: lane l owns value column (l & 15)
// and rows 4*(l >> 4) + i, i < 4.  The rows are the keys in a fixed order:
// inside each 32-row block, row 4g + i holds key 8g + i and row 16 + 4g + i holds
// key 8g + 4 + i (sigma below).  An accumulator tile pair (rows 32s..32s+31)
// then becomes a bf16 operand of a 16x16x32 MFMA directly, and lane group g
// carries the eight consecutive keys 32s + 8g .. 32s + 8g + 7 as its reduction
// slots, which is exactly a 16-byte read of a key-ordered LDS row.  So the
// q/k-side operands stay in natural key order (one 16-byte global load, one
// 16-byte LDS read per operand); only the state's load and store, the decay
// vector and the Kr tile (whose columns the state update reads as rows) follow
// the row order.  The A and B operands of the MFMA share one lane layout, so the
// same packed registers serve either side: P^T = Kc S^T takes S^T as B,
// O0 = S Qc^T takes it as A, which leaves O with four consecutive values of one
// token in each lane, ready for an 8-byte store.  The C-long reductions (U, the
// state update and the output) use the token analogue of the same slot order;
// with 16-token chunks the upper four slots of both operands are zero.  Every
// bf16 product uses the one 16x16x32 shape: a 16x16x16 MFMA that accumulates
// onto a 16x16x32 result was observed to read part of that accumulator before
// the first instruction had written it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kda_params.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
// The state side runs 2^-kStateExp below scale (see the header comment).
constexpr float kStateExp = 16.0f;
constexpr float kStateDown = 1.0f / 65536.0f;  // 2^-kStateExp
constexpr float kStateUp = 65536.0f;           // 2^kStateExp
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float((unsigned)x << 16); }
__device__ __forceinline__ float bflo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ u16 to_bf16(float x) { return (u16)(pack_bf16(x, 0.f) & 0xffffu); }

__device__ __forceinline__ f32x4_t mfma_k32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Workgroup barrier that orders LDS only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Makes one wave's LDS writes visible to the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// Key held by state row r (sigma in the header comment), and the row of key k.
__host__ __device__ constexpr int key_of_row(int r) {
  return (r & ~31) + (((r & 15) >> 2) << 3) + ((r & 16) ? 4 : 0) + (r & 3);
}
__host__ __device__ constexpr int row_of_key(int k) {
  return (k & ~31) + (((k & 31) >> 3) << 2) + ((k & 4) ? 16 : 0) + (k & 3);
}

template <int D_, int C_, int VT_, int NW_, int NSW_>
struct Cfg {
  static constexpr int D = D_;     // key = value head dimension
  static constexpr int C = C_;     // chunk length
  static constexpr int VT = VT_;   // value rows owned by the workgroup
  static constexpr int NW = NW_;   // waves
  static constexpr int NSW = NSW_; // waves 0..NSW-1 hold the state (and its MFMAs)
  static constexpr int NTHR = NW * 64;
  static constexpr int KT = D / 16;            // 16-row key tiles of S^T
  static constexpr int KS = D / 32;            // 32-wide steps of D-long reductions
  static constexpr int CT = C / 16;            // 16-row chunk tiles
  static constexpr int NTW = VT / (16 * NSW);  // 16-column value tiles per state wave
  // Role split: with at least four waves beyond the state waves, the state waves
  // also compute the whole gate and its prefix while the other waves (job waves)
  // run the chunk-local matrix jobs and stage the value tile; every wave takes a
  // share of the exponent-scaled operands.  The two roles run separate loops with
  // the same barriers.  With fewer waves every wave takes a share of everything
  // in one loop.
  static constexpr bool SPLIT = NW - NSW >= 4;
  // With at least eight job waves the state waves run the recurrence only: the gate,
  // the operands, the chunk matrices and the value tile are all the job waves' work,
  // one chunk further ahead (the state-only schedule).  A SIMD then holds one state
  // wave and two job waves, so the preparation's VALU work issues from two waves.
  static constexpr bool SO = NW - NSW >= 8;
  static constexpr int JOB_BASE = SPLIT ? NSW : 0;
  static constexpr int NJW = NW - JOB_BASE;      // job waves (they also stage v and beta)
  // gate waves: the state waves in the role split; the first four job waves in the
  // state-only schedule (the oldest, whom the issue arbiter serves first: the gate
  // is the job side's longest chain); job waves 4 and 5 take the two inversions
  static constexpr int NGW = SO ? 4 : (SPLIT ? NSW : NW);
  static constexpr int INV_BASE = 4;             // first inversion wave among the job waves
  static constexpr int NOW = SO ? NJW : NW;      // operand waves
  static constexpr int EPT = C * D / (NOW * 64);  // row layout (q, k; operand waves): positions per thread
  static constexpr int TPR = D / EPT;            // threads per chunk row
  static constexpr int EPV = C * VT / (NJW * 64);  // value row layout (job waves): elements per thread
  static constexpr int TPRV = VT / EPV;          // threads per value row
  static constexpr int SCOLS = D / NGW;          // column layout (g; gate waves): key columns per wave
  // A gate pass covers CPG column pairs by RG row groups (CPG * RG = 64 lanes): 16 x 4
  // when a wave has at least 32 columns, else 8 x 8.
  static constexpr int RG = SCOLS >= 32 ? 4 : 8;
  static constexpr int CPG = 64 / RG;
  static constexpr int SPASS = SCOLS / (2 * CPG);
  static constexpr int RPG = C / RG;             // chunk rows per row group
  static constexpr int LDQ = D + 16;           // bf16 row stride of [C][D] tiles (reads of
                                               // 16 rows x 4 lane groups are conflict-free)
  static constexpr int LDG = D + 4;            // fp32 row stride of the prefix tile
  static constexpr int LDR = D + 16;           // bf16 row stride of the [C][D] Kr tile
  static constexpr int LDC = C + 8;            // bf16 row stride of [C][C] tiles
  static constexpr int LDV = VT + 8;           // bf16 row stride of [C][VT] value tiles
  static constexpr int LDL = C + 4;            // fp32 row stride of [C][C] tiles
  static_assert(C == 16 || C == 32, "chunk");
  static_assert(NSW >= 1 && NSW <= NW, "state waves");
  static_assert(NTW >= 1 && NTW * 16 * NSW == VT, "value tiling");
  static_assert(EPT == 4 || EPT == 8 || EPT == 16, "row layout");
  static_assert(EPV == 4 || EPV == 8 || EPV == 16, "value row layout");
  static_assert(TPR >= 2 && TPR <= 32, "row reduction: DPP inside rows, one cross-row step");
  static_assert(SPASS >= 1 && SPASS * 2 * CPG * NGW == D, "column layout");
  static_assert(D % 32 == 0, "head dim");
  static_assert(NJW == 2 || NJW == 4 || NJW == 8, "job assignment");
  static_assert(!SO || NSW == 4, "state-only schedule: one state wave per SIMD");
  static_assert(C <= NJW * 64, "one beta per job thread");
};

// Job wave that runs chunk-local matrix job j (16x16 tiles; 32-token chunks:
// 0 L00, 1 L11, 2 L10, 3 Mqk10, 4 Mqk00, 5 Mqk11; 16-token chunks: 0 L00, 1 Mqk00).
// The two diagonal L jobs, which also invert their block, get waves of their own.
template <int NJW, int CT>
__device__ constexpr int job_wave(int j) {
  if (CT == 1) return j % NJW;
  if (NJW >= 6) return j;
  if (NJW == 4) return j < 4 ? j : j - 2;
  return j & 1;
}

// One chunk of one (sequence, head): its first token, its valid rows and its head.
struct Chunk {
  int64_t tok;
  int valid;
  int h;
};

// The centred operands Qc and Kc (key order), and Ki.  The state-only schedule
// writes the next chunk's while the state waves read the current chunk's, so they
// live in each slot there (Ki too, since the state waves form the chunk's matrix
// tiles in the step that uses them; the LDS-state mode has no room for a second Ki
// and forms them a step earlier); the other schedules keep one copy beside the slots.
template <class F, bool kHere>
struct QcKc {};
template <class F>
struct QcKc<F, true> {
  u16 Qc[F::C][F::LDQ];
  u16 Kc[F::C][F::LDQ];
};
template <class F, bool kHere>
struct KiBuf {};
template <class F>
struct KiBuf<F, true> {
  u16 Ki[F::C][F::LDQ];
};

// Prepared operands of one chunk.
template <class F, bool kKi>
struct alignas(16) Slot : QcKc<F, F::SO>, KiBuf<F, kKi> {
  u16 Kr[F::C][F::LDR];      // columns in state-row order (read transposed)
  u16 SOL[F::C][F::LDC];     // X11 2^-16, X22 2^-16 (X = (I + L)^-1 diagonal blocks) and
                             // -L21 2^16: the solve then yields U 2^-16
  u16 Mqk[F::C][F::LDC];      // 2^-Ca Mqk in two bf16 parts: Mqk, the nearest bf16, and
  u16 MqkLo[F::C][F::LDC];    // MqkLo, the nearest bf16 to the remainder
  u16 V[F::C][F::LDV];
  float a[2 * F::D];         // 2^G_T in state-row order (second half: discarded writes)
  float beta[F::C];          // sigmoid(beta), zero past the sequence
};

// The bf16 state of the LDS-state mode: rows are the workgroup's value rows, keys
// contiguous (the [V, K] layout of the state tensors), padded by 16 keys so that
// 16-byte reads of 16 rows fall in distinct banks.
template <class F, bool kHere>
struct StateLds {};
template <class F>
struct alignas(16) StateLds<F, true> {
  u16 Sb[F::VT][F::D + 16];
};

template <class F, int NSLOT, bool kSlds = false>
struct alignas(16) Smem : QcKc<F, !F::SO>, KiBuf<F, !F::SO || kSlds>, StateLds<F, kSlds> {  // (Qc, Kc: the chunk whose state side,
                             // matrices and preparation alternate in them)
  Slot<F, F::SO && !kSlds> slot[NSLOT];  // two alternate in the chunk loop; the prep
                                         // kernel uses one
  float G[F::C][F::LDG];     // inclusive base-2 decay prefix of the chunk being prepared,
                             // inside its row group of the gate layout
  float Goff[F::RG][F::D];   // ... plus this per row group and key: the prefix of the
                             // earlier row groups, minus the anchor
  float L[F::C][F::LDL];     // diagonal tiles of strictLower(diag(beta) Kc Ki^T)
  float gtc[2 * F::D];       // 2^(G_T - Ca) (second half: discarded writes)
  int pick;                  // the sequence this workgroup takes (automatic order)
};

// Stores N consecutive bf16 (N in {4, 8, 16}) from packed words.
template <int N>
__device__ __forceinline__ void store_words(u16* p, const unsigned* w) {
  if constexpr (N == 4) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{w[0], w[1]};
  } else {
#pragma unroll
    for (int h = 0; h < N / 8; ++h)
      *reinterpret_cast<u32x4_t*>(p + 8 * h) =
          u32x4_t{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
  }
}
// Stores N floats as bf16 (N in {4, 8, 16}).
template <int N>
__device__ __forceinline__ void store_bf16(u16* p, const float* x) {
  unsigned w[N / 2];
#pragma unroll
  for (int e = 0; e < N / 2; ++e) w[e] = pack_bf16(x[2 * e], x[2 * e + 1]);
  store_words<N>(p, w);
}

// Operand (16 rows x 32 reductions) of a 16x16x32 MFMA from a key-ordered bf16 LDS
// row: row r, columns k0 + 8g .. k0 + 8g + 7 (the reduction slots of lane group g).
__device__ __forceinline__ u32x4_t lds_op_k(const u16* row, int k0, int g) {
  return *reinterpret_cast<const u32x4_t*>(row + k0 + 8 * g);
}
// Operand from a naturally ordered [C][C] bf16 row with the pi_g permutation:
// columns 4g .. 4g+3 and 16 + 4g .. 16 + 4g + 3.
__device__ __forceinline__ u32x4_t lds_op_cc(const u16* row, int g) {
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row + 4 * g);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(row + 16 + 4 * g);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}
// Operand for a 16-long reduction: row r, columns 4g .. 4g+3, slots 4-7 zero.
__device__ __forceinline__ u32x4_t lds_op_pad(const u16* row, int g) {
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row + 4 * g);
  return u32x4_t{lo[0], lo[1], 0u, 0u};
}
// Transposed reads from a bf16 row-major [rows][ld] tile.  Inside each 16-lane
// group, lane i of a ds_read_b64_tr_b16 result takes element i%4 of the 4-element
// pieces addressed by lanes i/4, 4+i/4, 8+i/4 and 12+i/4; lane j addresses row
// 4g + j/4, columns k0 + 4(j%4) .. +3.  Lane i of group g so receives column
// k0 + i of rows 4g .. 4g+3.
__device__ __forceinline__ u32x2_t ds_read_tr(const u16* p) {
  return __builtin_bit_cast(
      u32x2_t,
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p)));
}
template <int LD>
__device__ __forceinline__ u32x2_t lds_col4(const u16* tile, int k0, int l16, int g) {
  return ds_read_tr(tile + (4 * g + (l16 >> 2)) * LD + k0 + 4 * (l16 & 3));
}
// Transposed operand: MFMA row m = column k0 + m, reduction slots = tile rows in
// pi_g order (4g + i, then 16 + 4g + i; upper slots zero when TWO is false).
template <int LD, bool TWO>
__device__ __forceinline__ u32x4_t lds_op_tr(const u16* tile, int k0, int l16, int g) {
  const u32x2_t lo = lds_col4<LD>(tile, k0, l16, g);
  if constexpr (TWO) {
    const u32x2_t hi = lds_col4<LD>(tile + 16 * LD, k0, l16, g);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return u32x4_t{lo[0], lo[1], 0u, 0u};
  }
}

// a.lo * b.lo + a.hi * b.hi + c for two packed bf16 pairs (fp32 accumulate).
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two accumulator tiles (rows 4g+i and 16+4g+i of one 32-row block) -> bf16 operand.
__device__ __forceinline__ u32x4_t acc_pair_to_op(f32x4_t t0, f32x4_t t1) {
  return u32x4_t{pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), pack_bf16(t1[0], t1[1]),
                 pack_bf16(t1[2], t1[3])};
}
// One accumulator tile (rows 4g+i of a 16-row block) -> bf16 operand, slots 4-7 zero.
__device__ __forceinline__ u32x4_t acc_to_op_pad(f32x4_t t0) {
  return u32x4_t{pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), 0u, 0u};
}

// Sum over aligned groups of G lanes (G in {2, 4, 8, 16, 32}) with DPP inside 16-lane rows:
// quad_perm xor 1, xor 2, then row_half_mirror (pairs quads) and row_mirror (pairs halves).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf,
                                                            0xf, false));
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16 || G == 32, "group size");
  v += dpp_f<0xB1>(v);                       // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_f<0x141>(v); // row_half_mirror
  if constexpr (G >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);  // across the two rows
  return v;
}

// Broadcast quad lane k's value to the four lanes of every quad (DPP quad_perm).
template <int K>
__device__ __forceinline__ float quad_bcast_k(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), K * 0x55,
                                                            0xf, 0xf, false));
}
__device__ __forceinline__ float quad_bcast(float v, int k) {
  switch (k) {
    case 0: return quad_bcast_k<0>(v);
    case 1: return quad_bcast_k<1>(v);
    case 2: return quad_bcast_k<2>(v);
    default: return quad_bcast_k<3>(v);
  }
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return zero
// and stores past it are dropped (third word: the gfx9 raw-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// Loads N consecutive bf16 (N in {4, 8, 16}) as packed words through a descriptor.
template <int N>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned* w) {
  if constexpr (N == 4) {
    const u32x2_t x = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    w[0] = x[0]; w[1] = x[1];
  } else {
#pragma unroll
    for (int hh = 0; hh < N / 8; ++hh) {
      const u32x4_t x =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * hh, 0, 0));
      w[4 * hh] = x[0]; w[4 * hh + 1] = x[1]; w[4 * hh + 2] = x[2]; w[4 * hh + 3] = x[3];
    }
  }
}

// Kernel modes: the fused forward; the split's token-parallel preparation (one
// chunk of one head per workgroup, written to the workspace as a record); the
// split's recurrent side (the fused schedule with every record read back instead
// of prepared).
constexpr int kModeFused = 0;
constexpr int kModePrep = 1;
constexpr int kModeRecur = 2;
// The fused forward with the state kept in LDS as bf16 between chunks and updated
// with fp32 arithmetic (FlashKDA's on-chip bf16 state, as "How FlashKDA Stores
// On-Chip Recurrent State in BF16 for Memory Efficiency" describes it): one
// rounding per chunk, state-only schedule only.
constexpr int kModeSlds = 3;

template <int D, int C, int VT, int NW, int NSW, int MODE>
__global__ __launch_bounds__(NW * 64) void kda_fwd_kernel(KdaParams p) {
  using F = Cfg<D, C, VT, NW, NSW>;
  static_assert(MODE == kModeFused || F::SPLIT, "the split runs the role-split schedules only");
  constexpr bool SLDS = MODE == kModeSlds;
  static_assert(!SLDS || F::SO, "the LDS state runs the state-only schedule only");
  __shared__ Smem<F, MODE == kModePrep ? 1 : 2, SLDS> sm;
  // the state waves form a chunk's matrix tiles in the step that uses them, from its
  // own copy of Ki (not in the LDS-state mode: one step earlier, from the one copy)
  constexpr bool kTilesLate = F::SO && !SLDS;
  using SlotT = Slot<F, kTilesLate>;
  // The centred operands of the chunk prepared in slot sl.
  auto qc_of = [&](SlotT& sl) -> u16(*)[F::LDQ] {
    if constexpr (F::SO) return sl.Qc;
    else return sm.Qc;
  };
  auto kc_of = [&](SlotT& sl) -> u16(*)[F::LDQ] {
    if constexpr (F::SO) return sl.Kc;
    else return sm.Kc;
  };
  auto ki_of = [&](SlotT& sl) -> u16(*)[F::LDQ] {
    if constexpr (kTilesLate) return sl.Ki;
    else return sm.Ki;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const bool is_state = wave < NSW;            // uniform per wave
  const bool is_job = wave >= F::JOB_BASE;     // uniform per wave
  const int jw = is_job ? wave - F::JOB_BASE : 0;        // index among the job waves
  const int jtid = is_job ? tid - F::JOB_BASE * 64 : 0;  // thread index among them

  // ---- work item (fused and recurrent kernels; the prep kernel maps slots) ---
  // Workgroups go to the eight XCDs round-robin by index, so blocks x and x + 8
  // share an XCD and its L2.  With several value tiles per (sequence, head), a
  // group of 8 * n_vtiles blocks holds eight units and gives the tiles of each to
  // blocks 8 apart: they read the same q, k and g, and the L2 serves all but the
  // first read.  Blocks past the last unit (padding of the last group) exit.
  // Start and end of sequence nn, clamped into [0, T_total].
  auto seq_bounds = [&](int nn, int64_t& a, int64_t& b) {
    if (p.cu != nullptr) {
      a = p.cu[nn];
      b = p.cu[nn + 1];
      a = a < 0 ? 0 : (a > p.T_total ? p.T_total : a);
      b = b < a ? a : (b > p.T_total ? p.T_total : b);
    } else {
      a = (int64_t)nn * p.T;
      b = a + p.T;
    }
  };
  int vt_idx = 0, h = 0, n = 0;
  int64_t s0 = 0, s1 = 0;
  int64_t rec0 = 0;  // split: the workspace slot of the work item's first chunk
  if constexpr (MODE == kModePrep) {
    // Block j * H + h prepares the chunk in slot j of head h.  Slots of sequence nn
    // start at floor(start(nn) / chunk_rows) + nn, which grows strictly with nn: a
    // bounded binary search finds the sequence; slots between sequences exit.
    h = (int)(blockIdx.x % (unsigned)p.H);
    const int64_t j = blockIdx.x / (unsigned)p.H;
    const int64_t CRl = p.chunk_rows;
    auto first_slot = [&](int nn) -> int64_t {
      int64_t a, b;
      seq_bounds(nn, a, b);
      return a / CRl + nn;
    };
    int lo = 0, hi = p.N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first_slot(mid) <= j) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
    int64_t a, b;
    seq_bounds(n, a, b);
    const int64_t c = j - (a / CRl + n);
    if (c < 0 || c * CRl >= b - a) return;  // uniform per workgroup
    s0 = a + c * CRl;
    s1 = s0 + CRl < b ? s0 + CRl : b;
    rec0 = j;
  } else {
    const int grp = 8 * p.n_vtiles;
    vt_idx = (int)(blockIdx.x % grp) / 8;
    const int unit = (int)(blockIdx.x / grp) * 8 + (int)(blockIdx.x % 8);
    if (unit >= p.N * p.H) return;  // uniform per workgroup
    h = unit % p.H;
    // Workgroups are dispatched in index order, so a caller's sequence order (for
    // example longest first) decides which sequences start first; it never changes
    // what a workgroup computes.  Entries are clamped into [0, N).
    n = unit / p.H;
    if (p.order != nullptr) {
      const int o = p.order[n];
      n = o < 0 ? 0 : (o >= p.N ? p.N - 1 : o);
    } else if (p.auto_order) {  // uniform
      // Longest first without a caller order (packed batches of at most
      // kMaxAutoOrderSeqs sequences whose workgroups outnumber the CUs): every
      // workgroup ranks the lengths, ties by index, and takes the sequence whose rank
      // is its slot.  Eight lanes share a candidate and sum its rank over their
      // share of the others; the prefix tile, not in use yet, holds the lengths.
      int* lens = reinterpret_cast<int*>(&sm.G[0][0]);
      for (int i = tid; i < p.N; i += F::NTHR) {
        const int64_t l = p.cu[i + 1] - p.cu[i];
        lens[i] = l < 0 ? 0 : (l > 0x7fffffff ? 0x7fffffff : (int)l);
      }
      lds_barrier();
      const int sub = lane & 7;
      for (int base = 0; base < p.N; base += F::NTHR / 8) {
        const int i = base + (tid >> 3);
        const int li = i < p.N ? lens[i] : 0;
        int r = 0;
        for (int j = sub; j < p.N; j += 8) {
          const int lj = lens[j];
          r += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        const float rank = group_sum<8>((float)r);  // exact: at most kMaxAutoOrderSeqs
        if (i < p.N && sub == 0 && (int)rank == n) sm.pick = i;
      }
      lds_barrier();
      n = sm.pick;
    }
    seq_bounds(n, s0, s1);
    if constexpr (MODE == kModeRecur) rec0 = s0 / p.chunk_rows + n;
  }
  const int64_t H = p.H;
  // Chunks of CR tokens; CR < C leaves the tile's last rows empty, which the ragged
  // tail handling already covers (zero inputs, no decay, no stores).
  const int CR = p.chunk_rows;
  const int nchunks = (int)((s1 - s0 + CR - 1) / CR);
  const uint32_t row_bytes = (uint32_t)(H * D * 2);
  const float Ca = p.anchor;
  const float c1 = __builtin_amdgcn_exp2f(Ca + kStateExp);  // 2^(Ca + 16): restores P
  const float c1o = c1 * p.scale;                           // ... and O, with the scale
  const float c1i = __builtin_amdgcn_exp2f(-Ca);            // 2^-Ca
  // tokens of the last chunk (uniform; every earlier chunk holds CR)
  const int last_valid = nchunks > 0 ? (int)(s1 - s0 - (int64_t)(nchunks - 1) * CR) : 0;
  auto chunk_valid = [&](int c) -> int { return c >= nchunks - 1 ? last_valid : CR; };
  auto ck = [&](int c) -> Chunk { return Chunk{s0 + (int64_t)c * CR, chunk_valid(c), h}; };
  const int64_t sbase0 = ((int64_t)n * H + h) * D * D;

  // ---- state: S^T accumulators of the state waves -----------------------------
  // Loaded and stored only inside the state waves' code paths, so no other wave
  // keeps registers for it.
  const int wv0 = wave * 16 * F::NTW;          // first value column of a state wave (in the tile)
  const int vbase = vt_idx * VT + wv0;         // ... in the head
  f32x4_t S[F::KT][F::NTW];
  // LDS-state mode: the chunk's decay in state-row order, read in phase A (in phase B
  // the gate waves overwrite the slot's decay vector with that of two chunks ahead)
  f32x4_t Adec[F::KT];
  // State I/O goes through a buffer descriptor based at the (sequence, head) state,
  // with one lane offset and a per-tile constant in the instruction's scalar offset
  // (no 64-bit address per tile).
  // Lane l16 of group lg handles value vbase + 16 nt + l16 and keys
  // key_of_row(16 kt + 4 lg) .. + 3 = 8 lg + kconst(kt) .. + 3.
  auto kconst = [](int kt) { return 32 * (kt >> 1) + 4 * (kt & 1); };
  // state_in issues the loads of the state's raw bits into the accumulators;
  // state_cvt widens them (bf16) and applies the 2^-16 state scale.
  auto state_in = [&](int64_t sbase) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) S[kt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (p.s_in == nullptr) return;
    const int es = p.s_in_fp32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(static_cast<const char*>(p.s_in) + sbase * es, D * D * es);
    if (p.s_kv) {
      // [K, V]: four element accesses per tile, coalesced across the lanes' values
      const uint32_t lo = (uint32_t)((8 * lg * D + vbase + l16) * es);
#pragma unroll
      for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ((kconst(kt) + i) * D + 16 * nt) * es;
            S[kt][nt][i] = p.s_in_fp32
                               ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, lo, c, 0))
                               : __uint_as_float(
                                     (unsigned)__builtin_amdgcn_raw_buffer_load_b16(rs, lo, c, 0));
          }
      return;
    }
    // [V, K]: 16-byte accesses.  The two tiles of a 32-row step hold keys 8 lg + 32 ks
    // .. + 3 and + 4 .. + 7 (the row order above), so in bf16 one access serves both.
    const uint32_t lo = (uint32_t)(((vbase + l16) * D + 8 * lg) * es);
    if (p.s_in_fp32) {
#pragma unroll
      for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
          S[kt][nt] = __builtin_bit_cast(
              f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lo, (16 * nt * D + kconst(kt)) * 4, 0));
      return;
    }
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        const u32x4_t w = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lo, (16 * nt * D + 32 * ks) * 2, 0));
        S[2 * ks][nt] = f32x4_t{__uint_as_float(w[0]), __uint_as_float(w[1]), 0.f, 0.f};
        S[2 * ks + 1][nt] = f32x4_t{__uint_as_float(w[2]), __uint_as_float(w[3]), 0.f, 0.f};
      }
  };
  auto state_cvt = [&]() __attribute__((always_inline)) {
    if (p.s_in == nullptr) return;
#pragma unroll
    for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        const f32x4_t r = S[kt][nt];
        if (p.s_in_fp32) {
          S[kt][nt] = kStateDown * r;
        } else if (p.s_kv) {
          // one bf16 per element, in the low half of its word
#pragma unroll
          for (int i = 0; i < 4; ++i) S[kt][nt][i] = kStateDown * bflo(__float_as_uint(r[i]));
        } else {
          const unsigned w0 = __float_as_uint(r[0]), w1 = __float_as_uint(r[1]);
          S[kt][nt] = kStateDown * f32x4_t{bflo(w0), bfhi(w0), bflo(w1), bfhi(w1)};
        }
      }
  };
  // The state is scaled back in place and stored tile by tile.
  auto state_out = [&](int64_t sbase) __attribute__((always_inline)) {
    if (p.s_out == nullptr) return;
    const int es = p.s_out_fp32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(static_cast<char*>(p.s_out) + sbase * es, D * D * es);
    if (p.s_kv) {
      const uint32_t lo = (uint32_t)((8 * lg * D + vbase + l16) * es);
#pragma unroll
      for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          S[kt][nt] = kStateUp * S[kt][nt];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ((kconst(kt) + i) * D + 16 * nt) * es;
            if (p.s_out_fp32)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[kt][nt][i]), rs, lo, c, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16(to_bf16(S[kt][nt][i]), rs, lo, c, 0);
          }
        }
      return;
    }
    const uint32_t lo = (uint32_t)(((vbase + l16) * D + 8 * lg) * es);
    if (p.s_out_fp32) {
#pragma unroll
      for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          S[kt][nt] = kStateUp * S[kt][nt];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, S[kt][nt]), rs, lo,
                                                 (16 * nt * D + kconst(kt)) * 4, 0);
        }
      return;
    }
    // bf16: one 16-byte store per tile pair (see state_in)
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        const f32x4_t a0 = kStateUp * S[2 * ks][nt], a1 = kStateUp * S[2 * ks + 1][nt];
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{pack_bf16(a0[0], a0[1]), pack_bf16(a0[2], a0[3]), pack_bf16(a1[0], a1[1]),
                    pack_bf16(a1[2], a1[3])},
            rs, lo, (16 * nt * D + 32 * ks) * 2, 0);
      }
  };

  // LDS-state mode: the state waves copy their value rows of the initial state into
  // the bf16 LDS state (rounded, and 2^16 below scale like the accumulators of the
  // register state) and back out at the end; eight keys per lane and access.
  constexpr int kSRowUnits = D / 8;                 // 8-key units per state row
  constexpr int kSUnits = 16 * F::NTW * kSRowUnits;  // units of a state wave's rows
  static_assert(kSUnits % 64 == 0, "state row units per lane");
  auto slds_in = [&](int64_t sbase) __attribute__((always_inline)) {
    if constexpr (SLDS) {
      const int es = p.s_in_fp32 ? 4 : 2;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(static_cast<const char*>(p.s_in) + sbase * es, D * D * es);
#pragma unroll
      for (int i = 0; i < kSUnits / 64; ++i) {
        const int u = lane + 64 * i;
        const int r = u / kSRowUnits, k0 = 8 * (u % kSRowUnits);
        const uint32_t off = (uint32_t)(((vbase + r) * D + k0) * es);
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (p.s_in != nullptr) {
          if (p.s_in_fp32) {
            const f32x4_t a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            const f32x4_t b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
          } else {
            const u32x4_t w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[2 * e] = bflo(w[e]); x[2 * e + 1] = bfhi(w[e]); }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= kStateDown;
        store_bf16<8>(&sm.Sb[wv0 + r][k0], x);
      }
    }
  };
  auto slds_out = [&](int64_t sbase) __attribute__((always_inline)) {
    if constexpr (SLDS) {
      if (p.s_out == nullptr) return;
      const int es = p.s_out_fp32 ? 4 : 2;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(static_cast<char*>(p.s_out) + sbase * es, D * D * es);
#pragma unroll
      for (int i = 0; i < kSUnits / 64; ++i) {
        const int u = lane + 64 * i;
        const int r = u / kSRowUnits, k0 = 8 * (u % kSRowUnits);
        const uint32_t off = (uint32_t)(((vbase + r) * D + k0) * es);
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(&sm.Sb[wv0 + r][k0]);
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = kStateUp * bflo(w[e]);
          x[2 * e + 1] = kStateUp * bfhi(w[e]);
        }
        if (p.s_out_fp32) {
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4_t, f32x4_t{x[0], x[1], x[2], x[3]}), rs, off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4_t, f32x4_t{x[4], x[5], x[6], x[7]}), rs, off + 16, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                      pack_bf16(x[6], x[7])},
              rs, off, 0, 0);
        }
      }
    }
  };

  // The block above the diagonal of Mqk is never written: zero it once.
  if constexpr (F::CT == 2) {
    constexpr int kSlots = MODE == kModePrep ? 1 : 2;
    for (int i = tid; i < kSlots * 16 * 16; i += F::NTHR) {
      const int b = i >> 8, r = (i >> 4) & 15, c = 16 + (i & 15);
      sm.slot[b].Mqk[r][c] = 0;
      sm.slot[b].MqkLo[r][c] = 0;
    }
  }

  // ======================= state side (state waves) ==========================
  f32x4_t P[F::CT][F::NTW], O[F::CT][F::NTW];
  // the value-tile columns of R, read at the start of phase A (state-only schedule)
  u32x2_t Vpre[F::CT][F::NTW];
  // A: P'^T = Kc S^T and O0' = S Qc^T (P = 2^Ca P', O0 = 2^Ca O0') with the decay
  // S^T <- diag(a) S^T alongside
  // (state_A), then R^T = diag(beta)(V - P^T) in place in P (state_R).
  auto state_A = [&](SlotT& cur) __attribute__((always_inline)) {
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (F::SO) {
      // R's value columns, read now so that their latency hides under the products
#pragma unroll
      for (int ct = 0; ct < F::CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
          Vpre[ct][nt] = lds_col4<F::LDV>(&cur.V[16 * ct][0], wv0 + 16 * nt, l16, lg);
    }
    // one 32-row key step at a time: its bf16 copy of S^T is live only there, and
    // once it is taken the decay of those rows proceeds while the products run
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks) {
      u32x4_t bS[F::NTW];
      if constexpr (SLDS) {
        // the bf16 state is the operand: keys 32 ks + 8 lg .. + 7 of value row l16
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
          bS[nt] = *reinterpret_cast<const u32x4_t*>(&sm.Sb[wv0 + 16 * nt + l16][32 * ks + 8 * lg]);
        Adec[2 * ks] = *reinterpret_cast<const f32x4_t*>(&cur.a[32 * ks + 4 * lg]);
        Adec[2 * ks + 1] = *reinterpret_cast<const f32x4_t*>(&cur.a[32 * ks + 16 + 4 * lg]);
      } else {
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
          bS[nt] = acc_pair_to_op(S[2 * ks][nt], S[2 * ks + 1][nt]);
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(&cur.a[32 * ks + 4 * lg]);
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(&cur.a[32 * ks + 16 + 4 * lg]);
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          S[2 * ks][nt] *= a0;
          S[2 * ks + 1][nt] *= a1;
        }
      }
#pragma unroll
      for (int ct = 0; ct < F::CT; ++ct) {
        const u32x4_t aK = lds_op_k(&kc_of(cur)[16 * ct + l16][0], 32 * ks, lg);
        const u32x4_t aQ = lds_op_k(&qc_of(cur)[16 * ct + l16][0], 32 * ks, lg);
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          P[ct][nt] = mfma_k32(aK, bS[nt], ks == 0 ? zero : P[ct][nt]);
          O[ct][nt] = mfma_k32(bS[nt], aQ, ks == 0 ? zero : O[ct][nt]);
        }
      }
    }
  };
  auto state_R = [&](SlotT& cur) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < F::CT; ++ct) {
      const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(&cur.beta[16 * ct + 4 * lg]);
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        // lane: value column wv0 + 16 nt + l16, chunk rows 16 ct + 4 lg .. +3
        u32x2_t vv;
        if constexpr (F::SO) vv = Vpre[ct][nt];
        else vv = lds_col4<F::LDV>(&cur.V[16 * ct][0], wv0 + 16 * nt, l16, lg);
        P[ct][nt][0] = b4[0] * __builtin_fmaf(-c1, P[ct][nt][0], bflo(vv[0]));
        P[ct][nt][1] = b4[1] * __builtin_fmaf(-c1, P[ct][nt][1], bfhi(vv[0]));
        P[ct][nt][2] = b4[2] * __builtin_fmaf(-c1, P[ct][nt][2], bflo(vv[1]));
        P[ct][nt][3] = b4[3] * __builtin_fmaf(-c1, P[ct][nt][3], bfhi(vv[1]));
      }
    }
  };
  // B: the blocked solve for U, the state update and the output of the current
  // chunk.  With INV = (I + L)^-1 = [[X11, 0], [X21, X22]] the solve U^T = INV R^T
  // runs as U_top = X11 R_top, U_bot = X22 (R_bot - L21 U_top), so X21 is never
  // formed; with the solve operands' power-of-two factors both halves come out
  // as U 2^-16, the state's own scale.  The output leaves as bf16 straight from
  // the accumulators, through a descriptor bounded to the chunk's valid rows.
  auto state_B = [&](SlotT& cur, const Chunk& ck) __attribute__((always_inline)) {
    u32x4_t bU[F::NTW];
    {
      const u32x4_t aX11 = lds_op_pad(&cur.SOL[l16][0], lg);
      f32x4_t Ut[F::NTW];
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt)
        Ut[nt] = mfma_k32(aX11, acc_to_op_pad(P[0][nt]), f32x4_t{0.f, 0.f, 0.f, 0.f});
      if constexpr (F::CT == 2) {
        const u32x4_t aNL21 = lds_op_pad(&cur.SOL[16 + l16][0], lg);
        const u32x4_t aX22 = lds_op_pad(&cur.SOL[16 + l16][16], lg);
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          const f32x4_t Tb = mfma_k32(aNL21, acc_to_op_pad(Ut[nt]), P[1][nt]);  // R_bot - L21 U_top
          const f32x4_t Ub = mfma_k32(aX22, acc_to_op_pad(Tb), f32x4_t{0.f, 0.f, 0.f, 0.f});
          bU[nt] = acc_pair_to_op(Ut[nt], Ub);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) bU[nt] = acc_to_op_pad(Ut[nt]);
      }
    }
    // O = 2^Ca (O0' + U Mqk'^T), Mqk' = 2^-Ca Mqk: U as the A operand (value rows),
    // Mqk' rows as B (token columns), Mqk' in its two bf16 parts (one product each).
    // Before the state update, so that O's accumulators are free while the update's
    // operands are read.
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(p.out + (ck.tok * H + ck.h) * D + vt_idx * VT, ck.valid * (int)row_bytes);
#pragma unroll
    for (int ct = 0; ct < F::CT; ++ct) {
      u32x4_t bM, bML;
      if constexpr (F::CT == 2) {
        bM = lds_op_cc(&cur.Mqk[16 * ct + l16][0], lg);
        bML = lds_op_cc(&cur.MqkLo[16 * ct + l16][0], lg);
      } else {
        bM = lds_op_pad(&cur.Mqk[l16][0], lg);
        bML = lds_op_pad(&cur.MqkLo[l16][0], lg);
      }
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        const f32x4_t o = c1o * mfma_k32(bU[nt], bML, mfma_k32(bU[nt], bM, O[ct][nt]));
        // lane: token 16 ct + l16, values wv0 + 16 nt + 4 lg .. +3
        const u32x2_t w = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
        __builtin_amdgcn_raw_buffer_store_b64(
            w, ro, (uint32_t)(16 * ct + l16) * row_bytes + (uint32_t)(wv0 + 16 * nt + 4 * lg) * 2,
            0, 0);
      }
    }
    // S^T += Kr^T U^T (the decay was applied in phase A).  LDS state: each 4-key
    // piece of the bf16 state is widened, decayed and accumulated in fp32, then
    // rounded back (one rounding per chunk).
#pragma unroll
    for (int kt = 0; kt < F::KT; ++kt) {
      const u32x4_t aR = lds_op_tr<F::LDR, F::CT == 2>(&cur.Kr[0][0], 16 * kt, l16, lg);
      if constexpr (SLDS) {
        // rows 16 kt + 4 lg + i hold keys key0 + i (the row order of the tiles)
        const f32x4_t av = Adec[kt];
        const int key0 = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1);
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          u16* ps = &sm.Sb[wv0 + 16 * nt + l16][key0];
          const u32x2_t w = *reinterpret_cast<const u32x2_t*>(ps);
          const f32x4_t t = av * f32x4_t{bflo(w[0]), bfhi(w[0]), bflo(w[1]), bfhi(w[1])};
          const f32x4_t u = mfma_k32(aR, bU[nt], t);
          *reinterpret_cast<u32x2_t*>(ps) = u32x2_t{pack_bf16(u[0], u[1]), pack_bf16(u[2], u[3])};
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) S[kt][nt] = mfma_k32(aR, bU[nt], S[kt][nt]);
      }
    }
  };

  // ======================= preparation ======================================
  // Column layout (g, gate, prefix; gate waves): pass ps covers key columns
  // g_col0 + 2 CPG ps and g_col0 + 2 CPG ps + 1 (lane % CPG picks the pair) and
  // chunk rows g_row0 .. g_row0 + RPG - 1 (lane / CPG picks one of RG row groups).
  const bool is_gate = F::SO ? (is_job && jw < F::NGW) : (!F::SPLIT || is_state);
  const int gw = F::SO ? (is_gate ? jw : 0)
                       : ((F::SPLIT && !is_state) ? 0 : wave);  // index among the gate waves
  const int g_col0 = gw * F::SCOLS + 2 * (lane % F::CPG);
  const int g_rg = lane / F::CPG;
  const int g_row0 = g_rg * F::RPG;
  // Row layout (q, k, operands; operand waves): chunk row r_row, positions r_col ..
  // r_col + EPT - 1.
  const int otid = F::SO ? jtid : tid;  // thread index among the operand waves
  const int r_row = otid / F::TPR;
  const int r_col = (otid % F::TPR) * F::EPT;
  // Value row layout (job waves).
  const int v_row = jtid / F::TPRV;
  const int v_col = (jtid % F::TPRV) * F::EPV;
  // Gate parameters of the head: the sigmoid argument in base 2 is gate_mul g + gate_add.
  float gate_mul, gate_add[F::SPASS][2];
  float raw_alog, raw_dtb[F::SPASS][2];
  auto load_gate_params = [&](int hh) {
    raw_alog = p.A_log[hh];
#pragma unroll
    for (int ps = 0; ps < F::SPASS; ++ps)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        raw_dtb[ps][c] = p.dt_bias[(int64_t)hh * D + g_col0 + 2 * F::CPG * ps + c];
  };
  auto set_gate_params = [&]() {
    gate_mul = -__expf(raw_alog) * kLog2e;
#pragma unroll
    for (int ps = 0; ps < F::SPASS; ++ps)
#pragma unroll
      for (int c = 0; c < 2; ++c) gate_add[ps][c] = gate_mul * raw_dtb[ps][c];
  };
  load_gate_params(h);
  set_gate_params();

  // Raw inputs of the chunk to prepare next, in registers.  Buffer loads through a
  // descriptor bounded to the chunk's valid rows: rows past the end of the
  // sequence read as zero, without branches.  Offsets are 32-bit (the host bounds
  // C * H * D * 2 below 2^31).
  const uint32_t off_qk = (uint32_t)r_row * row_bytes + (uint32_t)r_col * 2;
  const uint32_t off_v = (uint32_t)v_row * row_bytes + (uint32_t)(vt_idx * VT + v_col) * 2;
  const uint32_t off_g = (uint32_t)g_row0 * row_bytes + (uint32_t)g_col0 * 2;
  const uint32_t off_b = (uint32_t)jtid * (uint32_t)(H * 2);
  // Two register sets: the state-only schedule loads chunk c into set c % 2 a whole
  // step before it is used, while the other set is being consumed; the other
  // schedules use set 0 only.
  unsigned raw_q[2][F::EPT / 2], raw_k[2][F::EPT / 2];
  unsigned raw_v[2][F::EPV / 2];
  unsigned raw_g[2][F::SPASS][F::RPG];
  unsigned raw_b[2] = {0, 0};
  // g (gate waves), v and beta (job waves): consumed in phase A
  auto load_g = [&](const Chunk& ck, int b = 0) __attribute__((always_inline)) {
    const int64_t tok_elem = (ck.tok * H + ck.h) * D;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + tok_elem, ck.valid * (int)row_bytes);
#pragma unroll
    for (int ps = 0; ps < F::SPASS; ++ps)
#pragma unroll
      for (int i = 0; i < F::RPG; ++i)
        raw_g[b][ps][i] = __builtin_amdgcn_raw_buffer_load_b32(
            rg, off_g + (uint32_t)i * row_bytes + 4u * F::CPG * ps, 0, 0);
  };
  auto load_vb = [&](const Chunk& ck, int b = 0) __attribute__((always_inline)) {
    const int64_t tok_elem = (ck.tok * H + ck.h) * D;
    buf_load<F::EPV>(make_rsrc(p.v + tok_elem, ck.valid * (int)row_bytes), off_v, raw_v[b]);
    raw_b[b] = __builtin_amdgcn_raw_buffer_load_b16(
        make_rsrc(p.beta + ck.tok * H + ck.h, ck.valid * (int)H * 2), off_b, 0, 0);
  };
  // q and k: consumed in phase B
  auto load_qk = [&](const Chunk& ck, int b = 0) __attribute__((always_inline)) {
    const int64_t tok_elem = (ck.tok * H + ck.h) * D;
    const int nb = ck.valid * (int)row_bytes;
    buf_load<F::EPT>(make_rsrc(p.q + tok_elem, nb), off_qk, raw_q[b]);
    buf_load<F::EPT>(make_rsrc(p.k + tok_elem, nb), off_qk, raw_k[b]);
  };
  // Exclusive prefix over the row groups of a per-lane total t.  With four groups
  // each is one 16-lane row and the two lane swaps below combine them.  With eight
  // (lanes c, c+8, ..., c+56) row groups 2r and 2r+1 share the 16-lane row r: a DPP
  // shift by 8 inside the row gives the odd group its even neighbour, a rotate by 8
  // gives both the row total; the four row totals are then combined across rows
  // with the lane-swap instructions (the 16-row swap gives [r0, r0, r2, r2] and
  // [r1, r1, r3, r3]; their sum swapped across the 32-lane halves gives r0 + r1
  // to rows 2 and 3).
  auto rowgroup_excl = [&](float t) __attribute__((always_inline)) -> float {
    if constexpr (F::RG == 4) {
      // four row groups, one per 16-lane row: the lane swaps alone combine them
      const unsigned ab = __builtin_bit_cast(unsigned, t);
      const auto sw16 = __builtin_amdgcn_permlane16_swap(ab, ab, false, false);
      const float below = __builtin_bit_cast(float, (unsigned)sw16[0]);  // row r-1 for odd r
      const float pair = below + __builtin_bit_cast(float, (unsigned)sw16[1]);
      const unsigned pb = __builtin_bit_cast(unsigned, pair);
      const auto sw32 = __builtin_amdgcn_permlane32_swap(pb, pb, false, false);
      const float lower = __builtin_bit_cast(float, (unsigned)sw32[0]);  // r0 + r1
      return ((lg & 1) ? below : 0.f) + (lg >= 2 ? lower : 0.f);
    }
    const float in_row = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x118, 0xf, 0xf, true));
    const float rt = t + dpp_f<0x128>(t);
    const unsigned ab = __builtin_bit_cast(unsigned, rt);
    const auto sw16 = __builtin_amdgcn_permlane16_swap(ab, ab, false, false);
    const float below = __builtin_bit_cast(float, (unsigned)sw16[0]);  // row r-1 for odd r
    const float pair = below + __builtin_bit_cast(float, (unsigned)sw16[1]);
    const unsigned pb = __builtin_bit_cast(unsigned, pair);
    const auto sw32 = __builtin_amdgcn_permlane32_swap(pb, pb, false, false);
    const float lower = __builtin_bit_cast(float, (unsigned)sw32[0]);  // r0 + r1
    return in_row + ((lg & 1) ? below : 0.f) + (lg >= 2 ? lower : 0.f);
  };
  // A (gate waves): gate and inclusive prefix of the next chunk (column layout).
  auto gate_rows = [&](SlotT& nxt, int nxt_valid, auto full, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < F::SPASS; ++ps) {
      const int col = g_col0 + 2 * F::CPG * ps;
      // The sigmoids of all rows first, one instruction kind at a time (the rows are
      // independent, so each kind's latency is covered by the other rows), then the
      // running sums down the rows.
      float s0[F::RPG], s1[F::RPG];
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) {
        s0[i] = __builtin_fmaf(bflo(raw_g[b][ps][i]), gate_mul, gate_add[ps][0]);
        s1[i] = __builtin_fmaf(bfhi(raw_g[b][ps][i]), gate_mul, gate_add[ps][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(s0[i]);
        s1[i] = __builtin_amdgcn_exp2f(s1[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) {
        s0[i] = 1.0f + s0[i];
        s1[i] = 1.0f + s1[i];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) {
        s0[i] = __builtin_amdgcn_rcpf(s0[i]);
        s1[i] = __builtin_amdgcn_rcpf(s1[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
      float run0[F::RPG], run1[F::RPG];
      float t0 = 0.f, t1 = 0.f;
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) {
        if constexpr (decltype(full)::value) {
          t0 = __builtin_fmaf(p.lb2, s0[i], t0);
          t1 = __builtin_fmaf(p.lb2, s1[i], t1);
        } else {
          // no decay past the sequence; the floor only acts in one-token chunks
          const float lbv = g_row0 + i < nxt_valid ? p.lb2 : 0.f;
          t0 += __builtin_fmaxf(lbv * s0[i], p.lam2_floor);
          t1 += __builtin_fmaxf(lbv * s1[i], p.lam2_floor);
        }
        run0[i] = t0;
        run1[i] = t1;
      }
      const float off0 = rowgroup_excl(t0);
      const float off1 = rowgroup_excl(t1);
      // the prefix inside the row group, and the row group's offset (minus the
      // anchor) once per key: the operand preparation adds the two
#pragma unroll
      for (int i = 0; i < F::RPG; ++i)
        *reinterpret_cast<f32x2_t*>(&sm.G[g_row0 + i][col]) = f32x2_t{run0[i], run1[i]};
      *reinterpret_cast<f32x2_t*>(&sm.Goff[g_rg][col]) = f32x2_t{off0 - Ca, off1 - Ca};
      // G_T is the last row, held by the last row group; the other groups write the same
      // expressions into a discarded half of each array (no branch).  The decay
      // vector a goes to the state's row order (col is even, so the pair stays
      // adjacent), 2^(G_T - Ca) stays in key order.
      const float gt0 = t0 + off0, gt1 = t1 + off1;
      const int discard = (g_rg == F::RG - 1) ? 0 : F::D;
      *reinterpret_cast<f32x2_t*>(&nxt.a[discard + row_of_key(col)]) =
          f32x2_t{__builtin_amdgcn_exp2f(gt0), __builtin_amdgcn_exp2f(gt1)};
      *reinterpret_cast<f32x2_t*>(&sm.gtc[discard + col]) =
          f32x2_t{__builtin_amdgcn_exp2f(gt0 - Ca), __builtin_amdgcn_exp2f(gt1 - Ca)};
    }
  };
  // A (gate waves): gate and inclusive prefix of the next chunk (column layout);
  // a full chunk (the common case) skips the per-row end-of-sequence mask.
  auto gate = [&](SlotT& nxt, int nxt_valid, int b = 0) __attribute__((always_inline)) {
    if (nxt_valid == C) gate_rows(nxt, nxt_valid, std::true_type{}, b);
    else gate_rows(nxt, nxt_valid, std::false_type{}, b);
  };
  // A (job waves): value tile and beta of the next chunk.
  auto stage_vb = [&](SlotT& nxt, int nxt_valid, int b = 0) __attribute__((always_inline)) {
    store_words<F::EPV>(&nxt.V[v_row][v_col], raw_v[b]);
    if (jtid < C) nxt.beta[jtid] = jtid < nxt_valid ? fast_sigmoid(bf2f((u16)raw_b[b])) : 0.f;
  };
  // B: norms and exponent-scaled operands of the next chunk (keys r_col ..
  // r_col + EPT - 1 of chunk row r_row).
  auto prep_B = [&](SlotT& nxt, int b = 0) __attribute__((always_inline)) {
    // The prefix, offset and end factor of every position are read first (LDS reads
    // only, in flight while the norms reduce); then each arithmetic kind runs over all
    // positions, so the positions cover each other's latency; then the stores.
    constexpr int NG = F::EPT / 4;
    f32x4_t gg[NG], go[NG], tt[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int key = r_col + 4 * j;
      gg[j] = *reinterpret_cast<const f32x4_t*>(&sm.G[r_row][key]);
      go[j] = *reinterpret_cast<const f32x4_t*>(&sm.Goff[r_row / F::RPG][key]);
      tt[j] = *reinterpret_cast<const f32x4_t*>(&sm.gtc[key]);
    }
    float qn[F::EPT], kn[F::EPT];
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int w = 0; w < F::EPT / 2; ++w) {
      qn[2 * w] = bflo(raw_q[b][w]); qn[2 * w + 1] = bfhi(raw_q[b][w]);
      kn[2 * w] = bflo(raw_k[b][w]); kn[2 * w + 1] = bfhi(raw_k[b][w]);
      sq = dot2_bf16(raw_q[b][w], raw_q[b][w], sq);
      sk = dot2_bf16(raw_k[b][w], raw_k[b][w], sk);
    }
    sq = group_sum<F::TPR>(sq);
    sk = group_sum<F::TPR>(sk);
    const float rq = __builtin_amdgcn_rsqf(sq + kNormEps);
    const float rk = __builtin_amdgcn_rsqf(sk + kNormEps);
    float e1[F::EPT], e2[F::EPT];
#pragma unroll
    for (int x = 0; x < F::EPT; ++x) e1[x] = gg[x / 4][x % 4] + go[x / 4][x % 4];  // G - Ca
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < F::EPT; ++x) {
      e2[x] = __builtin_amdgcn_exp2f(-e1[x]);  // 2^(Ca - G)
      e1[x] = __builtin_amdgcn_exp2f(e1[x]);   // 2^(G - Ca)
    }
    __builtin_amdgcn_sched_barrier(0);
    float oQc[F::EPT], oKc[F::EPT], oKi[F::EPT], oKr[F::EPT];
#pragma unroll
    for (int x = 0; x < F::EPT; ++x) {
      const float qv = qn[x] * rq, kv = kn[x] * rk;
      oQc[x] = qv * e1[x];
      oKc[x] = kv * e1[x];
      oKi[x] = kv * e2[x];
      oKr[x] = oKi[x] * tt[x / 4][x % 4];  // kh 2^(G_T - G)
    }
    // eight positions (one 16-byte store per operand) at a time
    constexpr int RUN = F::EPT < 8 ? F::EPT : 8;
#pragma unroll
    for (int r0 = 0; r0 < F::EPT; r0 += RUN) {
#pragma unroll
      for (int j = 0; j < RUN / 4; ++j)
        store_bf16<4>(&nxt.Kr[r_row][row_of_key(r_col + r0 + 4 * j)], &oKr[r0 + 4 * j]);
      store_bf16<RUN>(&qc_of(nxt)[r_row][r_col + r0], &oQc[r0]);
      store_bf16<RUN>(&kc_of(nxt)[r_row][r_col + r0], &oKc[r0]);
      store_bf16<RUN>(&ki_of(nxt)[r_row][r_col + r0], &oKi[r0]);
    }
  };
  // A: the chunk-local matrices of the current chunk from its centred operands,
  // one 16x16 tile per job:
  //   L tiles:   L = strictLower(diag(beta) Kc Ki^T); a diagonal tile is inverted
  //              on the spot (X = (I + L)^-1), the lower-left tile is kept as -L21;
  //   Mqk tiles: lowerTri(Qc Ki^T).
  auto tile = [&](SlotT& cur, bool is_l, int ti, int tj) __attribute__((always_inline)) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const u16* arow = is_l ? &kc_of(cur)[16 * ti + l16][0] : &qc_of(cur)[16 * ti + l16][0];
    const u16* brow = &ki_of(cur)[16 * tj + l16][0];
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks)
      acc = mfma_k32(lds_op_k(arow, 32 * ks, lg), lds_op_k(brow, 32 * ks, lg), acc);
    const int j = 16 * tj + l16;
    if (!is_l) {
      // no contraction of the product into the remainder below: every kernel that
      // forms this tile (here and in the state waves' state_tile) then rounds alike,
      // whatever it knows of the tile's position at compile time
#pragma clang fp contract(off)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * ti + 4 * lg + ii;
        const float m = (j <= i) ? acc[ii] * c1i : 0.f;  // stored as 2^-Ca Mqk, in two parts
        const u16 hi = to_bf16(m);
        cur.Mqk[i][j] = hi;
        cur.MqkLo[i][j] = to_bf16(m - bf2f(hi));
      }
      return;
    }
    const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(&cur.beta[16 * ti + 4 * lg]);
    if (ti != tj) {
      // lower-left block: every entry is below the diagonal
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        cur.SOL[16 + 4 * lg + ii][j] = to_bf16(-kStateUp * b4[ii] * acc[ii]);
      return;
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * ti + 4 * lg + ii;
      sm.L[i][j] = (j < i) ? b4[ii] * acc[ii] : 0.f;
    }
    // forward substitution of the diagonal block, x_i = [i == m] - sum_{j<i} L_ij x_j
    // for every column m.  Column m lives in the lane quad 4m..4m+3; quad lane g
    // owns rows g, g+4, g+8, g+12 and holds those rows of L in registers.  At
    // step j the finished x_j is broadcast inside each quad (DPP quad_perm) and
    // every lane updates its four rows; L is zero on and above the diagonal, so
    // the update needs no masking.
    wave_lds_sync();
    const int base = 16 * ti;
    const int m = lane >> 2;
    const int gq = lane & 3;
    float Lr[4][16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j4 = 0; j4 < 16; j4 += 4) {
        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(&sm.L[base + gq + 4 * t][base + j4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) Lr[t][j4 + u] = w[u];
      }
    float x[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) x[t] = (gq + 4 * t == m) ? 1.f : 0.f;
#pragma unroll
    for (int jj = 0; jj < 15; ++jj) {
      const float xj = quad_bcast(x[jj >> 2], jj & 3);  // x_jj: quad lane jj%4, register jj/4
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = __builtin_fmaf(-Lr[t][jj], xj, x[t]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) cur.SOL[base + gq + 4 * t][base + m] = to_bf16(kStateDown * x[t]);
  };
  // The state waves' tile (job 2 + wave: L10, Mqk10, Mqk00, Mqk11) with its operand
  // rows chosen arithmetically, so that its reads and products share a block with
  // the state products; only the stores branch.
  auto state_tile = [&](SlotT& cur) __attribute__((always_inline)) {
    const bool t_l = wave == 0;
    const int t_i = wave == 2 ? 0 : 1;
    const int t_j = wave == 3 ? 1 : 0;
    const u16* arow = t_l ? &kc_of(cur)[16 * t_i + l16][0] : &qc_of(cur)[16 * t_i + l16][0];
    const u16* brow = &ki_of(cur)[16 * t_j + l16][0];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks)
      acc = mfma_k32(lds_op_k(arow, 32 * ks, lg), lds_op_k(brow, 32 * ks, lg), acc);
    const int j = 16 * t_j + l16;
    if (t_l) {
      const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(&cur.beta[16 + 4 * lg]);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        cur.SOL[16 + 4 * lg + ii][j] = to_bf16(-kStateUp * b4[ii] * acc[ii]);
    } else {
#pragma clang fp contract(off)  // as in tile()
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * t_i + 4 * lg + ii;
        const float m = (j <= i) ? acc[ii] * c1i : 0.f;
        const u16 hi = to_bf16(m);
        cur.Mqk[i][j] = hi;
        cur.MqkLo[i][j] = to_bf16(m - bf2f(hi));
      }
    }
  };
  // Matrix job j of a 32-token chunk: 0 L00, 1 L11 (each with its inversion), 2 L10,
  // 3 Mqk10, 4 Mqk00, 5 Mqk11.
  auto tile_job = [&](SlotT& cur, int j) __attribute__((always_inline)) {
    switch (j) {
      case 0: tile(cur, true, 0, 0); break;
      case 1: tile(cur, true, 1, 1); break;
      case 2: tile(cur, true, 1, 0); break;
      case 3: tile(cur, false, 1, 0); break;
      case 4: tile(cur, false, 0, 0); break;
      default: tile(cur, false, 1, 1); break;
    }
  };
  auto chunk_matrices = [&](SlotT& cur) __attribute__((always_inline)) {
    if constexpr (F::SO) {
      // the state-only schedule: the two inversions on job waves 4 and 5; the other
      // four tiles run on the state waves (see the state-only schedule below)
      if (jw >= F::INV_BASE && jw < F::INV_BASE + 2) tile_job(cur, jw - F::INV_BASE);
    } else if constexpr (F::CT == 2) {
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        if (job_wave<F::NJW, 2>(j) != jw) continue;  // uniform
        tile_job(cur, j);
      }
    } else {
      if (job_wave<F::NJW, 1>(0) == jw) tile(cur, true, 0, 0);
      if (job_wave<F::NJW, 1>(1) == jw) tile(cur, false, 0, 0);
    }
  };

  // ======================= split: prepared-chunk records ======================
  // A record is the byte image of what the state side reads from LDS for one
  // chunk: Qc, Kc, then Kr, SOL, Mqk (two parts) and a of its slot, in 16-byte
  // units.  The prep kernel stores it, the recurrent kernel's job waves load it one
  // chunk ahead (as q and k are loaded in the fused kernel) and copy it into LDS.
  constexpr int kQU = F::C * F::LDQ * 2 / 16;
  constexpr int kRU = F::C * F::LDR * 2 / 16;
  constexpr int kCU = F::C * F::LDC * 2 / 16;
  constexpr int kAU = F::D * 4 / 16;
  constexpr int kRecUnits = 2 * kQU + kRU + 3 * kCU + kAU;
  static_assert(kRecUnits * 16 == kda_record_bytes(D, C), "record layout");
  constexpr int kRecPerJob = (kRecUnits + F::NJW * 64 - 1) / (F::NJW * 64);
  auto rec_lds = [&](SlotT& sl, int u) -> u32x4_t* {
    char* b;
    int o;
    if (u < kQU) { b = reinterpret_cast<char*>(&qc_of(sl)[0][0]); o = u; }
    else if (u < 2 * kQU) { b = reinterpret_cast<char*>(&kc_of(sl)[0][0]); o = u - kQU; }
    else if (u < 2 * kQU + kRU) { b = reinterpret_cast<char*>(&sl.Kr[0][0]); o = u - 2 * kQU; }
    else if (u < 2 * kQU + kRU + kCU) {
      b = reinterpret_cast<char*>(&sl.SOL[0][0]);
      o = u - 2 * kQU - kRU;
    } else if (u < 2 * kQU + kRU + 2 * kCU) {
      b = reinterpret_cast<char*>(&sl.Mqk[0][0]);
      o = u - 2 * kQU - kRU - kCU;
    } else if (u < 2 * kQU + kRU + 3 * kCU) {
      b = reinterpret_cast<char*>(&sl.MqkLo[0][0]);
      o = u - 2 * kQU - kRU - 2 * kCU;
    } else {
      b = reinterpret_cast<char*>(&sl.a[0]);
      o = u - 2 * kQU - kRU - 3 * kCU;
    }
    return reinterpret_cast<u32x4_t*>(b + 16 * o);
  };
  // The head's workspace through a descriptor of its extent: an access past it
  // (only a malformed cu_seqlens can ask for one) reads zero or is dropped.
  auto ws_rsrc = [&]() {
    return make_rsrc(static_cast<char*>(p.ws) + (int64_t)h * p.ws_head_bytes,
                     (int)p.ws_head_bytes);
  };
  u32x4_t rec_raw[kRecPerJob];
  auto load_rec = [&](int c) {
    const __amdgpu_buffer_rsrc_t rw = ws_rsrc();
    const uint32_t base = (uint32_t)((rec0 + c) * (int64_t)(kRecUnits * 16));
#pragma unroll
    for (int i = 0; i < kRecPerJob; ++i) {
      const int u = jtid + F::NJW * 64 * i;
      if (u < kRecUnits)
        rec_raw[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, base + 16u * u, 0, 0));
    }
  };
  auto store_rec = [&](SlotT& sl) {
#pragma unroll
    for (int i = 0; i < kRecPerJob; ++i) {
      const int u = jtid + F::NJW * 64 * i;
      if (u < kRecUnits) *rec_lds(sl, u) = rec_raw[i];
    }
  };
  auto record_out = [&](SlotT& sl) {
    const __amdgpu_buffer_rsrc_t rw = ws_rsrc();
    const uint32_t base = (uint32_t)(rec0 * (int64_t)(kRecUnits * 16));
    for (int u = tid; u < kRecUnits; u += F::NTHR)
      __builtin_amdgcn_raw_buffer_store_b128(*rec_lds(sl, u), rw, base + 16u * u, 0, 0);
  };
  // beta alone (the prep kernel does not stage values)
  auto load_b = [&](const Chunk& ck) {
    raw_b[0] = __builtin_amdgcn_raw_buffer_load_b16(
        make_rsrc(p.beta + ck.tok * H + ck.h, ck.valid * (int)H * 2), off_b, 0, 0);
  };
  auto stage_b = [&](SlotT& nxt, int nxt_valid) {
    if (jtid < C) nxt.beta[jtid] = jtid < nxt_valid ? fast_sigmoid(bf2f((u16)raw_b[0])) : 0.f;
  };

  // ======================= schedule ==========================================
  // Step s: the state side of chunk s (A: P, O0, decay, R; B: solve, update,
  // output), the chunk-local matrices of chunk s (A) and the preparation of
  // chunk s+1 (A: gate, prefix, value tile; B: norms and operands); two
  // LDS-only barriers per step, the same count on every wave.
  const int c1st = nchunks > 1 ? 1 : 0;
  if constexpr (MODE == kModePrep) {
    // one chunk: gate (state waves) and beta (job waves), the operands (every
    // wave), the chunk-local matrices (job waves), then the record
    if (is_state) load_g(ck(0));
    else load_b(ck(0));
    load_qk(ck(0));
    if (is_state) gate(sm.slot[0], chunk_valid(0));
    else stage_b(sm.slot[0], chunk_valid(0));
    lds_barrier();
    prep_B(sm.slot[0]);
    lds_barrier();
    if (!is_state) chunk_matrices(sm.slot[0]);
    lds_barrier();
    record_out(sm.slot[0]);
  } else if constexpr (MODE == kModeRecur) {
    // the fused schedule's state side; the job waves stage the value tile and copy
    // the records in where the fused kernel prepares the chunk
    if (is_state) {
      state_in(sbase0);
      state_cvt();
      if (nchunks > 0) {
        lds_barrier();
        lds_barrier();
        for (int s = 0; s < nchunks; ++s) {
          SlotT& cur = sm.slot[s & 1];
          state_A(cur);
          state_R(cur);
          lds_barrier();
          state_B(cur, ck(s));
          lds_barrier();
        }
      }
      state_out(sbase0);
    } else if (nchunks > 0) {
      load_vb(ck(0));
      load_rec(0);
      stage_vb(sm.slot[0], chunk_valid(0));
      load_vb(ck(c1st));
      lds_barrier();
      store_rec(sm.slot[0]);
      load_rec(c1st);
      lds_barrier();
      for (int s = 0; s < nchunks; ++s) {
        SlotT& nxt = sm.slot[(s + 1) & 1];
        const bool more = s + 1 < nchunks;  // uniform
        const int nxt2 = s + 2 < nchunks ? s + 2 : nchunks - 1;
        if (more) {
          stage_vb(nxt, chunk_valid(s + 1));
          load_vb(ck(nxt2));
        }
        lds_barrier();
        if (more) {
          store_rec(nxt);
          load_rec(nxt2);
        }
        lds_barrier();
      }
    }
  } else if constexpr (F::SO) {
    // State-only schedule.  Step s: the state waves run chunk s (A: four of its matrix
    // tiles, P, O0, the decay and R; B: the solve, the state update and the output;
    // the LDS-state mode forms the four tiles of chunk s+1 at the end of B instead).
    // The job waves work one chunk further ahead: A: norms, operands and value tile
    // of chunk s+1; B: the two inverted tiles of chunk s+1 and the gate and prefix of
    // chunk s+2.  Three fill phases come first (gate of chunk 0; its operands; its
    // matrices and the gate of chunk 1); every wave passes the same barriers.
    if (is_state) {
      if constexpr (SLDS) {
        slds_in(sbase0);
      } else {
        state_in(sbase0);
        state_cvt();
      }
      if (nchunks > 0) {
        lds_barrier();
        lds_barrier();
        tile_job(sm.slot[0], 2 + wave);
        lds_barrier();
        for (int s = 0; s < nchunks; ++s) {
          SlotT& cur = sm.slot[s & 1];
          if (kTilesLate && s > 0) state_tile(cur);
          state_A(cur);
          state_R(cur);
          lds_barrier();
          state_B(cur, ck(s));
          if (!kTilesLate && s + 1 < nchunks) tile_job(sm.slot[(s + 1) & 1], 2 + wave);
          lds_barrier();
        }
      }
      if constexpr (SLDS) slds_out(sbase0);
      else state_out(sbase0);
    } else if (nchunks > 0) {
      // Raw inputs of chunk c go to register set c % 2, loaded at the start of the
      // phase a whole step before they are used.
      const int c2nd = nchunks > 2 ? 2 : nchunks - 1;
      if (is_gate) load_g(ck(0), 0);
      load_vb(ck(0), 0);
      load_qk(ck(0), 0);
      if (is_gate) load_g(ck(c1st), 1);
      load_vb(ck(c1st), 1);
      load_qk(ck(c1st), 1);
      if (is_gate) gate(sm.slot[0], chunk_valid(0), 0);
      stage_vb(sm.slot[0], chunk_valid(0), 0);
      lds_barrier();
      prep_B(sm.slot[0], 0);
      lds_barrier();
      if (is_gate) load_g(ck(c2nd), 0);
      chunk_matrices(sm.slot[0]);
      if (is_gate && nchunks > 1) gate(sm.slot[1], chunk_valid(1), 1);
      lds_barrier();
      // one step; b = s % 2 is a compile-time constant in the unrolled loop below
      auto job_step = [&](int s, auto par) __attribute__((always_inline)) {
        constexpr int b = decltype(par)::value;
        SlotT& nxt = sm.slot[(s + 1) & 1];
        const bool more = s + 1 < nchunks;   // uniform
        const bool more2 = s + 2 < nchunks;  // uniform
        const int n2 = more2 ? s + 2 : nchunks - 1;
        const int n3 = s + 3 < nchunks ? s + 3 : nchunks - 1;
        load_qk(ck(n2), b);
        load_vb(ck(n2), b);
        if (more) {
          prep_B(nxt, 1 - b);
          stage_vb(nxt, chunk_valid(s + 1), 1 - b);
        }
        lds_barrier();
        if (is_gate) load_g(ck(n3), 1 - b);
        if (more) chunk_matrices(nxt);
        if (more2 && is_gate) {
          // chunk s+2 goes to slot s % 2: its decay vector replaces chunk s's, which
          // the state waves read in phase A
          gate(sm.slot[s & 1], chunk_valid(s + 2), b);
        }
        lds_barrier();
      };
      for (int s = 0; s < nchunks; s += 2) {
        job_step(s, std::integral_constant<int, 0>{});
        if (s + 1 < nchunks) job_step(s + 1, std::integral_constant<int, 1>{});
      }
    }
  } else if constexpr (F::SPLIT) {
    if (is_state) {
      state_in(sbase0);
      state_cvt();
      if (nchunks > 0) {
        load_g(ck(0));
        load_qk(ck(0));
        gate(sm.slot[0], chunk_valid(0));
        load_g(ck(c1st));
        lds_barrier();
        prep_B(sm.slot[0]);
        load_qk(ck(c1st));
        lds_barrier();
        for (int s = 0; s < nchunks; ++s) {
          SlotT& cur = sm.slot[s & 1];
          SlotT& nxt = sm.slot[(s + 1) & 1];
          const bool more = s + 1 < nchunks;  // uniform
          const int nxt2 = s + 2 < nchunks ? s + 2 : nchunks - 1;
          state_A(cur);
          if (more) {
            gate(nxt, chunk_valid(s + 1));
            load_g(ck(nxt2));
          }
          state_R(cur);
          lds_barrier();
          state_B(cur, ck(s));
          if (more) {
            prep_B(nxt);
            load_qk(ck(nxt2));
          }
          lds_barrier();
        }
      }
      state_out(sbase0);
    } else if (nchunks > 0) {
      load_vb(ck(0));
      load_qk(ck(0));
      stage_vb(sm.slot[0], chunk_valid(0));
      load_vb(ck(c1st));
      lds_barrier();
      prep_B(sm.slot[0]);
      load_qk(ck(c1st));
      lds_barrier();
      for (int s = 0; s < nchunks; ++s) {
        SlotT& cur = sm.slot[s & 1];
        SlotT& nxt = sm.slot[(s + 1) & 1];
        const bool more = s + 1 < nchunks;  // uniform
        const int nxt2 = s + 2 < nchunks ? s + 2 : nchunks - 1;
        if (more) {
          stage_vb(nxt, chunk_valid(s + 1));
          load_vb(ck(nxt2));
        }
        chunk_matrices(cur);
        lds_barrier();
        if (more) {
          prep_B(nxt);
          load_qk(ck(nxt2));
        }
        lds_barrier();
      }
    }
  } else {
    if (is_state) {
      state_in(sbase0);
      state_cvt();
    }
    if (nchunks > 0) {
      load_g(ck(0));
      load_vb(ck(0));
      load_qk(ck(0));
      gate(sm.slot[0], chunk_valid(0));
      stage_vb(sm.slot[0], chunk_valid(0));
      load_g(ck(c1st));
      load_vb(ck(c1st));
      lds_barrier();
      prep_B(sm.slot[0]);
      load_qk(ck(c1st));
      lds_barrier();
      for (int s = 0; s < nchunks; ++s) {
        SlotT& cur = sm.slot[s & 1];
        SlotT& nxt = sm.slot[(s + 1) & 1];
        const bool more = s + 1 < nchunks;  // uniform
        const int nxt2 = s + 2 < nchunks ? s + 2 : nchunks - 1;
        if (is_state) state_A(cur);
        if (more) {
          gate(nxt, chunk_valid(s + 1));
          stage_vb(nxt, chunk_valid(s + 1));
          load_g(ck(nxt2));
          load_vb(ck(nxt2));
        }
        if (is_state) state_R(cur);
        chunk_matrices(cur);
        lds_barrier();
        if (is_state) state_B(cur, ck(s));
        if (more) {
          prep_B(nxt);
          load_qk(ck(nxt2));
        }
        lds_barrier();
      }
    }
    if (is_state) state_out(sbase0);
  }
}

template <int D, int C, int VT, int NW, int NSW, int MODE = kModeFused>
hipError_t launch_one(const KdaParams& p, hipStream_t stream) {
  // one block per unit with one value tile; otherwise whole groups of eight units;
  // the prep kernel: one block per workspace slot and head
  const int64_t units = (int64_t)p.N * p.H;
  const int64_t blocks =
      MODE == kModePrep ? kda_split_slots(p.T_total, p.N, p.chunk_rows) * p.H
      : p.n_vtiles == 1 ? units
                        : (units + 7) / 8 * 8 * p.n_vtiles;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kda_fwd_kernel<D, C, VT, NW, NSW, MODE>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// (D, chunk, value tile, waves, state waves)
#define KDA_SCHEDULES(X)  \
  X(128, 32, 128, 12, 4)  \
  X(128, 16, 128, 8, 4)   \
  X(128, 32, 64, 8, 4)    \
  X(128, 16, 64, 4, 4)    \
  X(64, 32, 64, 4, 4)     \
  X(64, 16, 64, 4, 4)     \
  X(64, 32, 32, 2, 2)     \
  X(64, 16, 32, 2, 2)     \
  X(32, 32, 32, 2, 2)     \
  X(32, 16, 32, 2, 2)

// Longest-first order of the sequences of a packed batch: one workgroup sorts the
// keys (kMaxInt - length) << 32 | index ascending with a bitonic network in LDS,
// so the longest sequence comes first and equal lengths keep their index order.
namespace {
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void kda_order_kernel(const int64_t* cu, int num_seqs,
                                                                   int padded, int32_t* order) {
  __shared__ uint64_t key[kMaxOrderSeqs];
  const int tid = threadIdx.x;
  for (int i = tid; i < padded; i += kOrderThreads) {
    uint64_t kv = ~0ull;  // padding sorts last
    if (i < num_seqs) {
      int64_t len = cu[i + 1] - cu[i];
      len = len < 0 ? 0 : (len > 0x7fffffff ? 0x7fffffff : len);
      kv = ((uint64_t)(0x7fffffff - len) << 32) | (uint32_t)i;
    }
    key[i] = kv;
  }
  __syncthreads();
  for (int size = 2; size <= padded; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < padded; i += kOrderThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t a = key[i], b = key[j];
          const bool ascending = (i & size) == 0;
          if ((a > b) == ascending) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < num_seqs; i += kOrderThreads) order[i] = (int32_t)(key[i] & 0xffffffffu);
}
}  // namespace

hipError_t launch_longest_first(const int64_t* cu, int num_seqs, int32_t* order,
                                hipStream_t stream) {
  if (num_seqs < 1 || num_seqs > kMaxOrderSeqs) return hipErrorInvalidValue;
  int padded = 1;
  while (padded < num_seqs) padded <<= 1;
  hipLaunchKernelGGL(kda_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, cu, num_seqs,
                     padded, order);
  return hipGetLastError();
}

bool kda_schedule_supported(int D, int chunk, int v_tile) { return kda_schedule_threads(D, chunk, v_tile) > 0; }

int kda_schedule_threads(int D, int chunk, int v_tile) {
#define KDA_THREADS(d, c, vt, nw, nsw) \
  if (D == d && chunk == c && v_tile == vt) return nw * 64;
  KDA_SCHEDULES(KDA_THREADS)
#undef KDA_THREADS
  return 0;
}

// The split's schedules: (D, chunk, value tile, waves, state waves) of the
// recurrent kernel; the prep kernel of a chunk length is the first of its row.
#define KDA_SPLIT_SCHEDULES(X) \
  X(128, 32, 128, 8, 4)        \
  X(128, 32, 64, 8, 4)         \
  X(128, 16, 128, 8, 4)

bool kda_split_supported(int D, int chunk, int v_tile) {
#define KDA_SPLIT_SUPPORTED(d, c, vt, nw, nsw) \
  if (D == d && chunk == c && v_tile == vt) return true;
  KDA_SPLIT_SCHEDULES(KDA_SPLIT_SUPPORTED)
#undef KDA_SPLIT_SUPPORTED
  return false;
}

hipError_t launch_kda_split(const KdaParams& p, int D, int chunk, int v_tile, hipStream_t stream) {
  if (!kda_split_supported(D, chunk, v_tile)) return hipErrorInvalidValue;
  hipError_t e = chunk == 32 ? launch_one<128, 32, 128, 8, 4, kModePrep>(p, stream)
                             : launch_one<128, 16, 128, 8, 4, kModePrep>(p, stream);
  if (e != hipSuccess) return e;
#define KDA_SPLIT_LAUNCH(d, c, vt, nw, nsw) \
  if (D == d && chunk == c && v_tile == vt) return launch_one<d, c, vt, nw, nsw, kModeRecur>(p, stream);
  KDA_SPLIT_SCHEDULES(KDA_SPLIT_LAUNCH)
#undef KDA_SPLIT_LAUNCH
  return hipErrorInvalidValue;
}

// The LDS-state mode's schedules (the state-only schedule at both value tiles).
#define KDA_SLDS_SCHEDULES(X) \
  X(128, 32, 128, 12, 4)      \
  X(128, 32, 64, 12, 4)

bool kda_slds_supported(int D, int chunk, int v_tile) {
#define KDA_SLDS_SUPPORTED(d, c, vt, nw, nsw) \
  if (D == d && chunk == c && v_tile == vt) return true;
  KDA_SLDS_SCHEDULES(KDA_SLDS_SUPPORTED)
#undef KDA_SLDS_SUPPORTED
  return false;
}

hipError_t launch_kda_fwd_slds(const KdaParams& p, int D, int chunk, int v_tile,
                               hipStream_t stream) {
#define KDA_SLDS_LAUNCH(d, c, vt, nw, nsw) \
  if (D == d && chunk == c && v_tile == vt) return launch_one<d, c, vt, nw, nsw, kModeSlds>(p, stream);
  KDA_SLDS_SCHEDULES(KDA_SLDS_LAUNCH)
#undef KDA_SLDS_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_kda_fwd(const KdaParams& p, int D, int chunk, int v_tile, hipStream_t stream) {
#define KDA_LAUNCH(d, c, vt, nw, nsw) \
  if (D == d && chunk == c && v_tile == vt) return launch_one<d, c, vt, nw, nsw>(p, stream);
  KDA_SCHEDULES(KDA_LAUNCH)
#undef KDA_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kda
