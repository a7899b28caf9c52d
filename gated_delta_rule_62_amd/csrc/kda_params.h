// Internal launch parameters shared by the host API and the HIP kernels.
#ifndef KDA_PARAMS_H_
#define KDA_PARAMS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct KdaParams {
  const uint16_t* q;        // bf16 [B*T, H, D]
  const uint16_t* k;        // bf16 [B*T, H, D]
  const uint16_t* v;        // bf16 [B*T, H, D]
  const uint16_t* g;        // bf16 [B*T, H, D]
  const uint16_t* beta;     // bf16 [B*T, H] (logits)
  uint16_t* out;            // bf16 [B*T, H, D]
  const float* A_log;       // [H]
  const float* dt_bias;     // [H, D]
  const void* s_in;         // [N, H, D, D] bf16/fp32 or nullptr
  void* s_out;              // [N, H, D, D] bf16/fp32 or nullptr
  const int64_t* cu;        // [N+1] or nullptr (batched)
  const int32_t* order;     // [N] sequence order of the workgroups, or nullptr (identity)
  int32_t auto_order;       // 1: no order given; the kernel dispatches longest first itself
  int64_t T;                // tokens per batch row (batched mode)
  int64_t T_total;          // B*T
  int32_t N;                // sequences
  int32_t H;                // heads
  int32_t s_in_fp32;        // 1: initial state is fp32
  int32_t s_out_fp32;       // 1: final state is fp32
  int32_t s_kv;             // 1: states are [N, H, K, V] (key-major) instead of [N, H, V, K]
  int32_t n_vtiles;         // value tiles per (sequence, head)
  int32_t chunk_rows;       // tokens per chunk: the tile height C, or fewer (1, 2, 4 or 8
                            // in a 16-row tile) to narrow each chunk's decay span
  float scale;              // output scale
  float lb2;                // lower_bound * log2(e)
  float lam2_floor;         // smallest per-token base-2 decay kept (-236 in one-token chunks
                            // when lb2 < -236, else -infinity: no floor)
  float anchor;             // fixed base-2 exponent anchor of the chunk
  // Two-kernel split only: the prepared-chunk workspace.  Head h owns ws_head_bytes
  // bytes at ws + h * ws_head_bytes, one record of kda_record_bytes(D, C) bytes per
  // slot; chunk c of sequence n sits in slot floor(start(n) / chunk_rows) + n + c.
  void* ws;
  int64_t ws_head_bytes;
};

// Bytes of one prepared-chunk record for head dimension D and tile height C: the
// byte images of the centred operands Qc and Kc ([C][D+16] bf16 each), the decayed
// keys Kr ([C][D+16] bf16), the solve operands and Mqk in two parts ([C][C+8] bf16
// each) and the chunk decay a (D fp32), as the recurrent side reads them from LDS.
constexpr int64_t kda_record_bytes(int64_t D, int64_t C) {
  return 2 * C * (D + 16) * 2 + C * (D + 16) * 2 + 3 * C * (C + 8) * 2 + D * 4;
}

// Slots per head of a split workspace: chunk starts never share a slot, and none
// exceeds floor(T_total / chunk_rows) + num_seqs.
constexpr int64_t kda_split_slots(int64_t T_total, int64_t num_seqs, int64_t chunk_rows) {
  return T_total / chunk_rows + num_seqs + 1;
}

// Launches the fused forward for a resolved schedule; returns a hipError_t.
hipError_t launch_kda_fwd(const KdaParams& p, int D, int chunk, int v_tile, hipStream_t stream);

// Whether a (D, chunk, v_tile) schedule has a compiled kernel.
bool kda_schedule_supported(int D, int chunk, int v_tile);

// Threads per workgroup of a compiled (D, chunk, v_tile) schedule, 0 if none.
int kda_schedule_threads(int D, int chunk, int v_tile);

// The LDS-state mode (bf16 state in LDS, fp32 update, one rounding per chunk):
// whether a schedule has a compiled kernel, and its launch.
bool kda_slds_supported(int D, int chunk, int v_tile);
hipError_t launch_kda_fwd_slds(const KdaParams& p, int D, int chunk, int v_tile,
                               hipStream_t stream);

// Threads per workgroup of the split's prep kernel.
constexpr int kSplitPrepThreads = 512;

// The two-kernel split: a token-parallel kernel writes every chunk's record into
// p.ws, then the recurrent kernel reads them back (same schedule as the fused
// kernel).  Both are enqueued on `stream`; returns a hipError_t.
hipError_t launch_kda_split(const KdaParams& p, int D, int chunk, int v_tile, hipStream_t stream);

// Whether the split has compiled kernels for a (D, chunk, v_tile) schedule.
bool kda_split_supported(int D, int chunk, int v_tile);

// Largest num_seqs the on-device longest-first ordering handles (one workgroup
// sorts all lengths in LDS).
constexpr int kMaxOrderSeqs = 8192;

// Largest num_seqs for which the forward kernel ranks the lengths itself.
constexpr int kMaxAutoOrderSeqs = 256;

// Launches the longest-first ordering of num_seqs (<= kMaxOrderSeqs) sequences.
hipError_t launch_longest_first(const int64_t* cu, int num_seqs, int32_t* order,
                                hipStream_t stream);

}  // namespace kda

#endif  // KDA_PARAMS_H_
