// Fused KDA recurrent prefill forward for gfx950 (CDNA4).
//
// One workgroup owns one (sequence n, head h, value tile j) work item and walks
// that sequence's chunks in order.  The fp32 state stays in MFMA accumulator
// registers for the whole sequence (the FlashInfer PR #4262 summary keeps it
// resident too, section 6, in tensor memory; here it is the accumulator file).
//
// Per chunk of C tokens (FlashInfer PR #4262 summary, sections 1-3):
//   1. load q, k, g, v, beta; L2-normalise q and k (scale folded into q);
//      gate lam2 = lb*log2(e)*sigmoid(exp(A_log)*(g + dt_bias)) (base 2)
//   2. inclusive prefix G over the chunk per key column; a = 2^G_T
//   3. operands (bf16, round to nearest even):
//        centred  Qc = qh 2^(G-Ca), Kc = kh 2^(G-Ca), Ki = kh 2^(Ca-G)
//        decayed  Qd = qh 2^G,      Kd = kh 2^G,      Kr = kh 2^(G_T-G)
//      with the fixed anchor Ca = (C/2) lb log2(e) (section 2: 16 b for C = 32)
//   4. L = strictLower(diag(beta) Kc Ki^T), Mqk = lowerTri(Qc Ki^T)  (bf16 MFMA,
//      masked by select so overflowed upper entries never propagate)
//   5. INV = (I + L)^-1 in fp32: forward substitution on 16x16 diagonal blocks,
//      the off-diagonal block by X21 = -X22 L21 X11 on fp32 MFMA
//   6. state side, per wave on its own value columns (section 3):
//        P^T = Kd S^T, O0^T = Qd S^T, R^T = diag(beta)(V - P^T), U^T = INV R^T,
//        S^T <- diag(a) S^T + Kr^T U^T,  O^T = O0^T + Mqk U^T
//
// Layout of the state in registers.  Each wave holds S^T (K rows x its value
// columns) as 16x16 fp32 accumulator tiles: lane l owns value column (l & 15)
// and key rows 4*(l >> 4) + i, i < 4.  An accumulator tile pair (key rows
// 32s..32s+31) becomes the bf16 B operand of a 16x16x32 MFMA directly: lane
// group g = l >> 4 then carries the reduction indices
//   pi_g = {32s + 4g + i} U {32s + 16 + 4g + i},  i < 4,
// and the A operands read from LDS use the same permutation, so the product is
// exact whatever order the hardware reduces in.  The same holds for the C-long
// reductions (U, the state update and the output) with the chunk tiles; with
// 16-token chunks the upper four slots of both operands are zero.  Every bf16
// product uses the one 16x16x32 shape: a 16x16x16 MFMA that accumulates onto
// a 16x16x32 result was observed to read part of that accumulator before the
// first instruction had written it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_params.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
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
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

template <int D_, int C_, int VT_, int NW_>
struct Cfg {
  static constexpr int D = D_;     // key = value head dimension
  static constexpr int C = C_;     // chunk length
  static constexpr int VT = VT_;   // value rows owned by the workgroup
  static constexpr int NW = NW_;   // waves
  static constexpr int NTHR = NW * 64;
  static constexpr int KT = D / 16;            // 16-row key tiles of S^T
  static constexpr int KS = D / 32;            // 32-wide steps of D-long reductions
  static constexpr int CT = C / 16;            // 16-row chunk tiles
  static constexpr int NTW = VT / (16 * NW);   // 16-column value tiles per wave
  static constexpr int EPT = C * D / NTHR;     // row-layout elements per thread
  static constexpr int TPR = D / EPT;          // threads per chunk row
  static constexpr int NGRP = NTHR / D;        // row groups of the column-layout scan
  static constexpr int RPG = C / NGRP;         // rows per scan group
  static constexpr int LDQ = D + 8;            // bf16 row stride of [C][D] tiles
  static constexpr int LDKT = C + 8;           // bf16 row stride of the [D][C] Kr^T tile
  static constexpr int LDC = C + 8;            // bf16 row stride of [C][C] tiles
  static constexpr int LDV = VT + 8;           // bf16 row stride of the [C][VT] value tile
  static constexpr int LDL = C + 4;            // fp32 row stride of [C][C] tiles
  static_assert(C == 16 || C == 32, "chunk");
  static_assert(NTW >= 1 && NTW * 16 * NW == VT, "value tiling");
  static_assert(EPT == 4 || EPT == 8 || EPT == 16, "row layout");
  static_assert(TPR <= 64 && (64 % TPR) == 0, "row reduction stays inside a wave");
  static_assert(NGRP >= 1 && C % NGRP == 0, "scan layout");
  static_assert(D % 32 == 0, "head dim");
};

template <class F>
struct alignas(16) Smem {
  u16 Qc[F::C][F::LDQ];
  u16 Kc[F::C][F::LDQ];
  u16 Ki[F::C][F::LDQ];
  u16 Qd[F::C][F::LDQ];
  u16 Kd[F::C][F::LDQ];
  u16 KrT[F::D][F::LDKT];
  u16 V[F::C][F::LDV];
  u16 INV[F::C][F::LDC];
  u16 Mqk[F::C][F::LDC];
  float G[F::C][F::D];       // base-2 decay, then its inclusive prefix
  float L[F::C][F::LDL];     // strictLower(diag(beta) Kc Ki^T)
  float X[F::C][F::LDL];     // fp32 (I + L)^-1
  float Y[16][17];           // L21 X11 of the blocked inverse
  float tot[F::NGRP][F::D];  // scan group totals
  float a[F::D];             // 2^G_T
  float gtc[F::D];           // 2^(G_T - Ca)
  float beta[F::C];          // sigmoid(beta)
};

// Loads N consecutive bf16 as floats (N in {4, 8, 16}); p is 8- or 16-byte aligned.
template <int N>
__device__ __forceinline__ void load_bf16(const u16* p, float* out) {
  if constexpr (N == 4) {
    u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
    out[0] = bflo(w[0]); out[1] = bfhi(w[0]); out[2] = bflo(w[1]); out[3] = bfhi(w[1]);
  } else {
#pragma unroll
    for (int h = 0; h < N / 8; ++h) {
      u32x4_t w = *reinterpret_cast<const u32x4_t*>(p + 8 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[8 * h + 2 * e] = bflo(w[e]);
        out[8 * h + 2 * e + 1] = bfhi(w[e]);
      }
    }
  }
}

// Stores N floats as bf16 to LDS (N in {4, 8, 16}).
template <int N>
__device__ __forceinline__ void store_bf16(u16* p, const float* x) {
  if constexpr (N == 4) {
    u32x2_t w = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    *reinterpret_cast<u32x2_t*>(p) = w;
  } else {
#pragma unroll
    for (int h = 0; h < N / 8; ++h) {
      u32x4_t w = {pack_bf16(x[8 * h], x[8 * h + 1]), pack_bf16(x[8 * h + 2], x[8 * h + 3]),
                   pack_bf16(x[8 * h + 4], x[8 * h + 5]), pack_bf16(x[8 * h + 6], x[8 * h + 7])};
      *reinterpret_cast<u32x4_t*>(p + 8 * h) = w;
    }
  }
}

// A operand (16 rows x 32 reductions) of a 16x16x32 MFMA read from a bf16 row-major
// LDS tile with the pi_g permutation: row r, columns k0 + 4g .. +3 and k0 + 16 + 4g .. +3.
__device__ __forceinline__ u32x4_t lds_a_pi(const u16* row, int k0, int g) {
  u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row + k0 + 4 * g);
  u32x2_t hi = *reinterpret_cast<const u32x2_t*>(row + k0 + 16 + 4 * g);
  u32x4_t r = {lo[0], lo[1], hi[0], hi[1]};
  return r;
}

// Two accumulator tiles (rows 4g+i and 16+4g+i of one 32-row block) -> bf16 B operand.
__device__ __forceinline__ u32x4_t acc_pair_to_b(f32x4_t t0, f32x4_t t1) {
  u32x4_t r = {pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), pack_bf16(t1[0], t1[1]),
               pack_bf16(t1[2], t1[3])};
  return r;
}
// One accumulator tile (rows 4g+i of a 16-row block) -> bf16 B operand whose
// reduction slots 4-7 are zero.
__device__ __forceinline__ u32x4_t acc_to_b_pad(f32x4_t t0) {
  u32x4_t r = {pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), 0u, 0u};
  return r;
}
// A operand for a 16-long reduction: row r, columns 4g .. 4g+3, slots 4-7 zero.
__device__ __forceinline__ u32x4_t lds_a_pad(const u16* row, int g) {
  u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row + 4 * g);
  u32x4_t r = {lo[0], lo[1], 0u, 0u};
  return r;
}

template <int D, int C, int VT, int NW>
__global__ __launch_bounds__(NW * 64) void kda_fwd_kernel(KdaParams p) {
  using F = Cfg<D, C, VT, NW>;
  __shared__ Smem<F> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // ---- work item ---------------------------------------------------------
  const int vt_idx = blockIdx.x % p.n_vtiles;
  const int unit = blockIdx.x / p.n_vtiles;
  const int h = unit % p.H;
  const int n = unit / p.H;
  int64_t s0, s1;
  if (p.cu != nullptr) {
    s0 = p.cu[n];
    s1 = p.cu[n + 1];
    s0 = s0 < 0 ? 0 : (s0 > p.T_total ? p.T_total : s0);
    s1 = s1 < s0 ? s0 : (s1 > p.T_total ? p.T_total : s1);
  } else {
    s0 = (int64_t)n * p.T;
    s1 = s0 + p.T;
  }
  const int64_t H = p.H;

  // ---- per-head constants ------------------------------------------------
  const float A = __expf(p.A_log[h]);
  const int r_row = tid / F::TPR;              // chunk row of the row layout
  const int r_col = (tid % F::TPR) * F::EPT;   // first key column of the row layout
  float gate_mul = -A * kLog2e;                // sigmoid argument in base 2
  float gate_add[F::EPT];
#pragma unroll
  for (int e = 0; e < F::EPT; ++e) gate_add[e] = gate_mul * p.dt_bias[(int64_t)h * D + r_col + e];
  const float Ca = p.anchor;
  const float c1 = __builtin_amdgcn_exp2f(Ca);  // 2^Ca

  // ---- state in: S^T accumulators ----------------------------------------
  const int vbase = vt_idx * VT + wave * 16 * F::NTW;  // first value row of this wave
  f32x4_t S[F::KT][F::NTW];
  {
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        const int vrow = vbase + 16 * nt + l16;
        const int kcol = 16 * kt + 4 * lg;
        const int64_t off = sbase + (int64_t)vrow * D + kcol;
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
        if (p.s_in != nullptr) {
          if (p.s_in_fp32) {
            s = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p.s_in) + off);
          } else {
            u32x2_t w = *reinterpret_cast<const u32x2_t*>(static_cast<const u16*>(p.s_in) + off);
            s[0] = bflo(w[0]); s[1] = bfhi(w[0]); s[2] = bflo(w[1]); s[3] = bfhi(w[1]);
          }
        }
        S[kt][nt] = s;
      }
  }

  // Zero the fp32 inverse once: blocks above the diagonal are never written.
  for (int i = tid; i < F::C * F::LDL; i += F::NTHR) (&sm.X[0][0])[i] = 0.f;
  // Zero the upper 16x16 block of Mqk once (C = 32): it is never written.
  if constexpr (F::CT == 2) {
    for (int i = tid; i < 16 * 16; i += F::NTHR) sm.Mqk[i / 16][16 + i % 16] = 0;
  }

  for (int64_t c0 = s0; c0 < s1; c0 += C) {
    const int valid = (s1 - c0) < C ? (int)(s1 - c0) : C;

    // ---- 1. loads, norms, gate (row layout) ------------------------------
    float qv[F::EPT], kv[F::EPT];
    {
      const bool rv = r_row < valid;
      float gv[F::EPT];
      if (rv) {
        const int64_t off = ((c0 + r_row) * H + h) * D + r_col;
        load_bf16<F::EPT>(p.q + off, qv);
        load_bf16<F::EPT>(p.k + off, kv);
        load_bf16<F::EPT>(p.g + off, gv);
      } else {
#pragma unroll
        for (int e = 0; e < F::EPT; ++e) { qv[e] = 0.f; kv[e] = 0.f; gv[e] = 0.f; }
      }
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < F::EPT; ++e) {
        sq = __builtin_fmaf(qv[e], qv[e], sq);
        sk = __builtin_fmaf(kv[e], kv[e], sk);
      }
#pragma unroll
      for (int m = 1; m < F::TPR; m <<= 1) {
        sq += __shfl_xor(sq, m, 64);
        sk += __shfl_xor(sk, m, 64);
      }
      const float rq = p.scale * __builtin_amdgcn_rsqf(sq + kNormEps);
      const float rk = __builtin_amdgcn_rsqf(sk + kNormEps);
      float lam[F::EPT];
#pragma unroll
      for (int e = 0; e < F::EPT; ++e) {
        qv[e] *= rq;
        kv[e] *= rk;
        const float sg = __builtin_amdgcn_rcpf(
            1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(gv[e], gate_mul, gate_add[e])));
        lam[e] = rv ? p.lb2 * sg : 0.f;
      }
#pragma unroll
      for (int e = 0; e < F::EPT; e += 4) {
        f32x4_t w = {lam[e], lam[e + 1], lam[e + 2], lam[e + 3]};
        *reinterpret_cast<f32x4_t*>(&sm.G[r_row][r_col + e]) = w;
      }
    }
    // value tile (16-byte pieces)
    for (int pc = tid; pc < C * VT / 8; pc += F::NTHR) {
      const int row = pc / (VT / 8);
      const int col = (pc % (VT / 8)) * 8;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (row < valid)
        w = *reinterpret_cast<const u32x4_t*>(p.v + ((c0 + row) * H + h) * D + vt_idx * VT + col);
      *reinterpret_cast<u32x4_t*>(&sm.V[row][col]) = w;
    }
    if (tid < C) sm.beta[tid] = tid < valid ? fast_sigmoid(bf2f(p.beta[(c0 + tid) * H + h])) : 0.f;
    __syncthreads();

    // ---- 2. inclusive prefix over the chunk (column layout) ----------------
    {
      const int col = tid % D;
      const int grp = tid / D;
      float run[F::RPG];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) {
        acc += sm.G[grp * F::RPG + i][col];
        run[i] = acc;
      }
      sm.tot[grp][col] = acc;
      __syncthreads();
      float off = 0.f;
#pragma unroll
      for (int gg = 0; gg < F::NGRP - 1; ++gg)
        if (gg < grp) off += sm.tot[gg][col];
#pragma unroll
      for (int i = 0; i < F::RPG; ++i) sm.G[grp * F::RPG + i][col] = run[i] + off;
      if (grp == F::NGRP - 1) {
        const float gt = acc + off;
        sm.a[col] = __builtin_amdgcn_exp2f(gt);
        sm.gtc[col] = __builtin_amdgcn_exp2f(gt - Ca);
      }
    }
    __syncthreads();

    // ---- 3. exponent-scaled operands (row layout) ---------------------------
    {
      float oQc[F::EPT], oKc[F::EPT], oKi[F::EPT], oQd[F::EPT], oKd[F::EPT];
#pragma unroll
      for (int e = 0; e < F::EPT; ++e) {
        const float d = sm.G[r_row][r_col + e] - Ca;
        const float e1 = __builtin_amdgcn_exp2f(d);   // 2^(G - Ca)
        const float e2 = __builtin_amdgcn_exp2f(-d);  // 2^(Ca - G)
        const float ed = e1 * c1;                     // 2^G
        oQc[e] = qv[e] * e1;
        oKc[e] = kv[e] * e1;
        oKi[e] = kv[e] * e2;
        oQd[e] = qv[e] * ed;
        oKd[e] = kv[e] * ed;
        sm.KrT[r_col + e][r_row] = to_bf16(oKi[e] * sm.gtc[r_col + e]);  // kh 2^(G_T - G)
      }
      store_bf16<F::EPT>(&sm.Qc[r_row][r_col], oQc);
      store_bf16<F::EPT>(&sm.Kc[r_row][r_col], oKc);
      store_bf16<F::EPT>(&sm.Ki[r_row][r_col], oKi);
      store_bf16<F::EPT>(&sm.Qd[r_row][r_col], oQd);
      store_bf16<F::EPT>(&sm.Kd[r_row][r_col], oKd);
    }
    __syncthreads();

    // ---- 4. intra-chunk products: L and Mqk (bf16 MFMA) ---------------------
    {
      constexpr int NTRI = F::CT * (F::CT + 1) / 2;
      for (int job = wave; job < 2 * NTRI; job += NW) {
        const int which = job / NTRI;  // 0: L, 1: Mqk
        const int tri = job % NTRI;
        const int ti = tri == 0 ? 0 : (tri == 1 ? 1 : 1);
        const int tj = tri == 0 ? 0 : (tri == 1 ? 0 : 1);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const u16* arow = which ? &sm.Qc[16 * ti + l16][0] : &sm.Kc[16 * ti + l16][0];
        const u16* brow = &sm.Ki[16 * tj + l16][0];
#pragma unroll
        for (int s = 0; s < F::KS; ++s) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(arow + 32 * s + 8 * lg);
          u32x4_t b = *reinterpret_cast<const u32x4_t*>(brow + 32 * s + 8 * lg);
          acc = mfma_k32(a, b, acc);
        }
        const int j = 16 * tj + l16;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * ti + 4 * lg + ii;
          if (which == 0) {
            sm.L[i][j] = (j < i) ? sm.beta[i] * acc[ii] : 0.f;
          } else {
            sm.Mqk[i][j] = to_bf16((j <= i) ? acc[ii] : 0.f);
          }
        }
      }
    }
    __syncthreads();

    // ---- 5. INV = (I + L)^-1 (fp32) ------------------------------------------
    if (wave == 0) {
      // diagonal 16x16 blocks by forward substitution: lane m of block b owns
      // column m of that block; x_i = [i == m] - sum_{j < i} L_ij x_j inside it.
      const int m = lane & 15;
      const int base = (F::CT == 2) ? 16 * ((lane >> 4) & 1) : 0;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == m) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) s = __builtin_fmaf(-sm.L[base + i][base + j], x[j], s);
        x[i] = s;
      }
      if (lane < C) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.X[base + i][base + m] = x[i];
      }
    }
    __syncthreads();
    if constexpr (F::CT == 2) {
      // X21 = -X22 (L21 X11) on the fp32 MFMA: lane l supplies A[l&15][k] and
      // B[k][l&15] with k = 4s + (l >> 4); results come back in accumulator layout.
      if (wave == 0) {
        f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kk = 4 * s + lg;
          y = mfma_f32(sm.L[16 + l16][kk], sm.X[kk][l16], y);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sm.Y[4 * lg + ii][l16] = y[ii];
      }
      __syncthreads();
      if (wave == 0) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kk = 4 * s + lg;
          z = mfma_f32(sm.X[16 + l16][16 + kk], sm.Y[kk][l16], z);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sm.X[16 + 4 * lg + ii][l16] = -z[ii];
      }
      __syncthreads();
    }
    for (int i = tid; i < C * C; i += F::NTHR) sm.INV[i / C][i % C] = to_bf16(sm.X[i / C][i % C]);
    __syncthreads();

    // ---- 6. state side (each wave: its value columns) -----------------------
    {
      // B operands from the bf16 copy of S^T
      u32x4_t bS[F::KS][F::NTW];
#pragma unroll
      for (int s = 0; s < F::KS; ++s)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) bS[s][nt] = acc_pair_to_b(S[2 * s][nt], S[2 * s + 1][nt]);

      f32x4_t P[F::CT][F::NTW], O[F::CT][F::NTW];
#pragma unroll
      for (int ct = 0; ct < F::CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) {
          P[ct][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          O[ct][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ct = 0; ct < F::CT; ++ct)
#pragma unroll
        for (int s = 0; s < F::KS; ++s) {
          const u32x4_t aK = lds_a_pi(&sm.Kd[16 * ct + l16][0], 32 * s, lg);
          const u32x4_t aQ = lds_a_pi(&sm.Qd[16 * ct + l16][0], 32 * s, lg);
#pragma unroll
          for (int nt = 0; nt < F::NTW; ++nt) {
            P[ct][nt] = mfma_k32(aK, bS[s][nt], P[ct][nt]);
            O[ct][nt] = mfma_k32(aQ, bS[s][nt], O[ct][nt]);
          }
        }

      // R^T = diag(beta) (V - P^T), in place in P
#pragma unroll
      for (int ct = 0; ct < F::CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int c = 16 * ct + 4 * lg + ii;
            const int vc = wave * 16 * F::NTW + 16 * nt + l16;
            P[ct][nt][ii] = sm.beta[c] * (bf2f(sm.V[c][vc]) - P[ct][nt][ii]);
          }

      // U^T = INV R^T, then the bf16 B operands of U^T
      f32x4_t U[F::CT][F::NTW];
      if constexpr (F::CT == 2) {
        u32x4_t bR[F::NTW];
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) bR[nt] = acc_pair_to_b(P[0][nt], P[1][nt]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const u32x4_t aI = lds_a_pi(&sm.INV[16 * ct + l16][0], 0, lg);
#pragma unroll
          for (int nt = 0; nt < F::NTW; ++nt)
            U[ct][nt] = mfma_k32(aI, bR[nt], f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
        u32x4_t bU[F::NTW];
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) bU[nt] = acc_pair_to_b(U[0][nt], U[1][nt]);
        // S^T <- diag(a) S^T + Kr^T U^T
#pragma unroll
        for (int kt = 0; kt < F::KT; ++kt) {
          f32x4_t av = *reinterpret_cast<const f32x4_t*>(&sm.a[16 * kt + 4 * lg]);
          const u32x4_t aR = lds_a_pi(&sm.KrT[16 * kt + l16][0], 0, lg);
#pragma unroll
          for (int nt = 0; nt < F::NTW; ++nt) {
            S[kt][nt] = S[kt][nt] * av;
            S[kt][nt] = mfma_k32(aR, bU[nt], S[kt][nt]);
          }
        }
        // O^T = O0^T + Mqk U^T
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const u32x4_t aM = lds_a_pi(&sm.Mqk[16 * ct + l16][0], 0, lg);
#pragma unroll
          for (int nt = 0; nt < F::NTW; ++nt) O[ct][nt] = mfma_k32(aM, bU[nt], O[ct][nt]);
        }
      } else {
        // 16-token chunks: the same 16x16x32 instruction with reduction slots 4-7
        // zero in both operands (one MFMA shape on every accumulator chain).
        u32x4_t bR[F::NTW];
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) bR[nt] = acc_to_b_pad(P[0][nt]);
        const u32x4_t aI = lds_a_pad(&sm.INV[l16][0], lg);
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
          U[0][nt] = mfma_k32(aI, bR[nt], f32x4_t{0.f, 0.f, 0.f, 0.f});
        u32x4_t bU[F::NTW];
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) bU[nt] = acc_to_b_pad(U[0][nt]);
#pragma unroll
        for (int kt = 0; kt < F::KT; ++kt) {
          f32x4_t av = *reinterpret_cast<const f32x4_t*>(&sm.a[16 * kt + 4 * lg]);
          const u32x4_t aR = lds_a_pad(&sm.KrT[16 * kt + l16][0], lg);
#pragma unroll
          for (int nt = 0; nt < F::NTW; ++nt) {
            S[kt][nt] = S[kt][nt] * av;
            S[kt][nt] = mfma_k32(aR, bU[nt], S[kt][nt]);
          }
        }
        const u32x4_t aM = lds_a_pad(&sm.Mqk[l16][0], lg);
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt) O[0][nt] = mfma_k32(aM, bU[nt], O[0][nt]);
      }

      // store O^T -> out[token, h, value] (bf16)
#pragma unroll
      for (int ct = 0; ct < F::CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < F::NTW; ++nt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int c = 16 * ct + 4 * lg + ii;
            if (c < valid) {
              const int64_t off = ((c0 + c) * H + h) * D + vbase + 16 * nt + l16;
              p.out[off] = to_bf16(O[ct][nt][ii]);
            }
          }
    }
    __syncthreads();
  }

  // ---- state out ------------------------------------------------------------
  if (p.s_out != nullptr) {
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
    for (int kt = 0; kt < F::KT; ++kt)
#pragma unroll
      for (int nt = 0; nt < F::NTW; ++nt) {
        const int vrow = vbase + 16 * nt + l16;
        const int kcol = 16 * kt + 4 * lg;
        const int64_t off = sbase + (int64_t)vrow * D + kcol;
        const f32x4_t s = S[kt][nt];
        if (p.s_out_fp32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.s_out) + off) = s;
        } else {
          u32x2_t w = {pack_bf16(s[0], s[1]), pack_bf16(s[2], s[3])};
          *reinterpret_cast<u32x2_t*>(static_cast<u16*>(p.s_out) + off) = w;
        }
      }
  }
}

template <int D, int C, int VT, int NW>
hipError_t launch_one(const KdaParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.N * p.H * p.n_vtiles;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kda_fwd_kernel<D, C, VT, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

#define KDA_SCHEDULES(X)  \
  X(128, 32, 128, 4)      \
  X(128, 16, 128, 4)      \
  X(128, 32, 64, 4)       \
  X(128, 16, 64, 4)       \
  X(64, 32, 64, 4)        \
  X(64, 16, 64, 4)        \
  X(64, 32, 32, 2)        \
  X(64, 16, 32, 2)        \
  X(32, 32, 32, 2)        \
  X(32, 16, 32, 2)

bool kda_schedule_supported(int D, int chunk, int v_tile) {
#define KDA_SUPPORTED(d, c, vt, nw) \
  if (D == d && chunk == c && v_tile == vt) return true;
  KDA_SCHEDULES(KDA_SUPPORTED)
#undef KDA_SUPPORTED
  return false;
}

hipError_t launch_kda_fwd(const KdaParams& p, int D, int chunk, int v_tile, hipStream_t stream) {
#define KDA_LAUNCH(d, c, vt, nw) \
  if (D == d && chunk == c && v_tile == vt) return launch_one<d, c, vt, nw>(p, stream);
  KDA_SCHEDULES(KDA_LAUNCH)
#undef KDA_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kda
