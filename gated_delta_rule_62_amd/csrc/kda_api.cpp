// Host side of the C ABI declared in include/kda.h: argument validation,
// schedule selection and the kernel launch.  Nothing here touches device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/kda.h"
#include "kda_params.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;
// Largest decay span (base 2) of a chunk.  The operands are centred on the middle
// of the span, so they reach at most 2^(span/2) = 2^118 (|qh|, |kh| <= 1): 2^9
// below the bf16 maximum, and the smallest of them, 2^-118 times a component,
// keeps 8 binades above the bf16 normal minimum for the components' own range.
constexpr double kMaxSpan = 236.0;

struct Range {
  uintptr_t lo;
  uintptr_t hi;  // exclusive
};

Range make_range(const void* p, int64_t bytes) {
  Range r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (bytes > 0 ? static_cast<uintptr_t>(bytes) : 0);
  return r;
}

bool overlaps(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;  // empty ranges never overlap
  return a.lo < b.hi && b.lo < a.hi;
}

// Decay span (base 2) of a chunk: the largest magnitude of its prefix, chunk |lb| log2(e).
double chunk_span(double lb, int chunk) { return chunk * std::fabs(lb) * kLog2e; }

bool chunk_admissible(double lb, int chunk) { return chunk_span(lb, chunk) <= kMaxSpan; }

// Tokens per chunk: 32 or 16 fill a 32- or 16-row tile; 8, 4, 2 and 1 run in a
// 16-row tile whose last rows stay empty, which narrows the chunk's decay span for
// strongly negative lower bounds.
bool chunk_rows_valid(int rows) {
  return rows == 32 || rows == 16 || rows == 8 || rows == 4 || rows == 2 || rows == 1;
}
int tile_rows(int rows) { return rows == 32 ? 32 : 16; }

// One-token chunks admit every lower bound: past |lb| = 236 / log2(e) = 163.6 the
// kernel floors the per-token base-2 decay at -236 (a factor below 1e-71).
bool rows_admissible(double lb, int rows) { return rows == 1 || chunk_admissible(lb, rows); }
bool needs_decay_floor(double lb, int rows) { return rows == 1 && !chunk_admissible(lb, 1); }

// The longest admissible chunk.
int auto_chunk(double lb) {
  for (int rows = 32; rows > 1; rows /= 2)
    if (chunk_admissible(lb, rows)) return rows;
  return 1;
}

// Compute units of the current device (256 on MI355X when the query fails, e.g.
// without a GPU).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

// One workgroup owns all value rows of a (sequence, head) unless there are so few
// units that halving the value tile still leaves one workgroup per compute unit:
// the halves repeat the chunk preparation but split the state work.
int auto_v_tile(int64_t D, int chunk, int64_t units) {
  if (D == 128 && chunk == 32 && 2 * units <= device_cus()) return 64;
  return static_cast<int>(D);
}

int resolve(const void* q, const void* k, const void* v, const void* g, const void* beta,
            float scale, const void* out, const float* A_log, const float* dt_bias,
            float lower_bound, const void* initial_state, int initial_state_dtype,
            const void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
            int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, int chunk_size,
            int v_tile, const int32_t* seq_order, int* chunk_out, int* v_tile_out) {
  // With no tokens (every sequence empty) the kernels touch no activation buffer, so
  // those pointers may be NULL, as a zero-element tensor's are.
  const bool tokens = B > 0 && T > 0;
  if ((tokens && (!q || !k || !v || !g || !beta || !out)) || !A_log || !dt_bias)
    return KDA_ERR_NULL_ARG;
  if (B < 1 || H < 1 || T < 0) return KDA_ERR_BAD_SHAPE;
  if (T == 0 && cu_seqlens == nullptr) return KDA_ERR_BAD_SHAPE;
  if (D != 32 && D != 64 && D != 128) return KDA_ERR_BAD_SHAPE;
  // The kernels address one chunk (up to 32 token rows) with 32-bit byte offsets:
  // H * D * 64 < 2^31.  Every size test is a division, so no product of caller
  // sizes is formed before it is known to fit (64 D divides 2^31 exactly).
  if (H >= ((int64_t)1 << 31) / (64 * D) || T > ((int64_t)1 << 40) / B) return KDA_ERR_BAD_SHAPE;
  // activation extents below 2^62 bytes, so the range arithmetic cannot wrap
  if (B * T > ((int64_t)1 << 62) / (H * D * 2)) return KDA_ERR_BAD_SHAPE;
  if (initial_state && initial_state_dtype != KDA_DTYPE_BF16 &&
      initial_state_dtype != KDA_DTYPE_FP32)
    return KDA_ERR_BAD_DTYPE;
  if (final_state && final_state_dtype != KDA_DTYPE_BF16 && final_state_dtype != KDA_DTYPE_FP32)
    return KDA_ERR_BAD_DTYPE;
  if (cu_seqlens) {
    if (B != 1 || num_seqs < 1) return KDA_ERR_BAD_VARLEN;
  } else {
    if (num_seqs != B) return KDA_ERR_BAD_VARLEN;
  }
  if (num_seqs > (((int64_t)1 << 31) / 4) / H) return KDA_ERR_BAD_SHAPE;  // num_seqs H <= 2^29
  if (!std::isfinite(scale)) return KDA_ERR_BAD_SCALE;
  if (!std::isfinite(lower_bound) || !(lower_bound < 0.f)) return KDA_ERR_BAD_LOWER_BOUND;

  // lb log2(e) must be a finite fp32 value (|lb| below 2.35e38)
  if (!std::isfinite(static_cast<float>(lower_bound * kLog2e))) return KDA_ERR_BAD_LOWER_BOUND;

  int chunk = chunk_size == 0 ? auto_chunk(lower_bound) : chunk_size;
  if (!chunk_rows_valid(chunk)) return KDA_ERR_BAD_SCHEDULE;
  if (!rows_admissible(lower_bound, chunk)) return KDA_ERR_BAD_LOWER_BOUND;
  const int tile = tile_rows(chunk);
  int vt = v_tile == 0 ? auto_v_tile(D, tile, num_seqs * H) : v_tile;
  if (!kda::kda_schedule_supported(static_cast<int>(D), tile, vt)) return KDA_ERR_BAD_SCHEDULE;
  // One launch covers at most 2^32 - 1 work-items: workgroups (units rounded up to
  // groups of eight when a unit has several value tiles) times their threads.
  const int64_t tiles = D / vt;
  const int64_t groups = tiles == 1 ? num_seqs * H : (num_seqs * H + 7) / 8 * 8 * tiles;
  if (groups > (((int64_t)1 << 32) - 1) / kda::kda_schedule_threads(static_cast<int>(D), tile, vt))
    return KDA_ERR_BAD_SHAPE;

  // Buffer extents and the aliasing contract.
  const int64_t tok = B * T;
  const int64_t act = tok * H * D * 2;
  const int64_t st_elems = num_seqs * H * D * D;
  const Range rq = make_range(q, act), rk = make_range(k, act), rv = make_range(v, act),
              rg = make_range(g, act), rb = make_range(beta, tok * H * 2),
              ra = make_range(A_log, H * 4), rd = make_range(dt_bias, H * D * 4),
              rc = make_range(cu_seqlens, cu_seqlens ? (num_seqs + 1) * 8 : 0),
              ro = make_range(seq_order, seq_order ? num_seqs * 4 : 0),
              rs_in = make_range(initial_state,
                                 initial_state ? st_elems * (initial_state_dtype ? 4 : 2) : 0),
              rout = make_range(out, act),
              rs_out = make_range(final_state,
                                  final_state ? st_elems * (final_state_dtype ? 4 : 2) : 0);
  const Range inputs_but_state[] = {rq, rk, rv, rg, rb, ra, rd, rc, ro};
  for (const Range& r : inputs_but_state) {
    if (overlaps(rout, r) || overlaps(rs_out, r)) return KDA_ERR_BAD_ALIAS;
  }
  if (overlaps(rout, rs_in) || overlaps(rout, rs_out)) return KDA_ERR_BAD_ALIAS;
  if (overlaps(rs_out, rs_in)) {
    const bool exact = initial_state == final_state && initial_state_dtype == final_state_dtype;
    if (!exact) return KDA_ERR_BAD_ALIAS;
  }
  *chunk_out = chunk;
  *v_tile_out = vt;
  return KDA_OK;
}

// Bytes of the split's workspace per head for a resolved chunk length, or a negative
// status: the split runs D = 128 only, and every record offset and the prep grid
// must fit 31 bits.
int64_t split_head_bytes(int64_t T_total, int64_t num_seqs, int64_t H, int64_t D, int chunk) {
  if (D != 128) return KDA_ERR_BAD_SCHEDULE;
  const int64_t slots = kda::kda_split_slots(T_total, num_seqs, chunk);
  const int64_t rec = kda::kda_record_bytes(D, tile_rows(chunk));
  if (slots > (((int64_t)1 << 31) - 1) / rec || slots > (((int64_t)1 << 31) - 1) / H)
    return KDA_ERR_BAD_SHAPE;
  // the prep kernel's grid (one workgroup per slot and head) stays below 2^32 work-items
  if (slots * H > (((int64_t)1 << 32) - 1) / kda::kSplitPrepThreads) return KDA_ERR_BAD_SHAPE;
  return slots * rec;
}

// Scratch of kda_fwd_split_noalloc: the split's workspace in a device array that
// every GPU the library runs on holds until the process ends.  Host code never uses
// the array's name as an address: the address of each device's copy is resolved
// once, with that device current, and kept per device.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The current device's scratch address, or a negative status.
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return KDA_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return KDA_OK;
}

// Validates, fills the launch parameters and enqueues the kernel, or with a
// workspace (split) the prep and recurrent kernels.
int launch(const void* q, const void* k, const void* v, const void* g, const void* beta,
           float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
           const void* initial_state, int initial_state_dtype, void* final_state,
           int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
           int64_t T, int64_t H, int64_t D, void* stream, int chunk_size, int v_tile,
           const int32_t* seq_order, int state_kv, bool split = false, void* workspace = nullptr,
           int64_t workspace_bytes = 0, bool lds_state = false) {
  int chunk = 0, vt = 0;
  const int st = resolve(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                         initial_state, initial_state_dtype, final_state, final_state_dtype,
                         cu_seqlens, num_seqs, B, T, H, D, chunk_size, v_tile, seq_order, &chunk,
                         &vt);
  if (st != KDA_OK) return st;
  if (lds_state && !kda::kda_slds_supported(static_cast<int>(D), tile_rows(chunk), vt))
    return KDA_ERR_BAD_SCHEDULE;
  int64_t head_bytes = 0;
  if (split) {
    if (!kda::kda_split_supported(static_cast<int>(D), tile_rows(chunk), vt))
      return KDA_ERR_BAD_SCHEDULE;
    head_bytes = split_head_bytes(B * T, num_seqs, H, D, chunk);
    if (head_bytes < 0) return static_cast<int>(head_bytes);
    if (!workspace) return KDA_ERR_NULL_ARG;
    if (workspace_bytes < head_bytes * H) return KDA_ERR_BAD_WORKSPACE;
    // the workspace is written: it must not overlap any argument buffer
    const int64_t act = B * T * H * D * 2;
    const int64_t st_elems = num_seqs * H * D * D;
    const Range rw = make_range(workspace, head_bytes * H);
    const Range others[] = {
        make_range(q, act), make_range(k, act), make_range(v, act), make_range(g, act),
        make_range(beta, B * T * H * 2), make_range(A_log, H * 4), make_range(dt_bias, H * D * 4),
        make_range(cu_seqlens, cu_seqlens ? (num_seqs + 1) * 8 : 0), make_range(out, act),
        make_range(initial_state, initial_state ? st_elems * (initial_state_dtype ? 4 : 2) : 0),
        make_range(final_state, final_state ? st_elems * (final_state_dtype ? 4 : 2) : 0)};
    for (const Range& r : others) {
      if (overlaps(rw, r)) return KDA_ERR_BAD_ALIAS;
    }
  }

  kda::KdaParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g);
  p.beta = static_cast<const uint16_t*>(beta);
  p.out = static_cast<uint16_t*>(out);
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.s_in = initial_state;
  p.s_out = final_state;
  p.cu = cu_seqlens;
  p.order = seq_order;
  // Without a caller order, a packed batch whose workgroups outnumber the CUs by up
  // to four times (so a few start only when others finish, and a long one starting
  // last would set the time) is dispatched longest first by the kernel.  With more
  // workgroups the dispatch already balances itself and the ranking would only cost.
  const int64_t grid = num_seqs * H * (D / vt);
  const int64_t cus = device_cus();
  p.auto_order = (cu_seqlens != nullptr && seq_order == nullptr &&
                  num_seqs <= kda::kMaxAutoOrderSeqs && grid > cus && grid <= 4 * cus)
                     ? 1
                     : 0;
  p.T = T;
  p.T_total = B * T;
  p.N = static_cast<int32_t>(num_seqs);
  p.H = static_cast<int32_t>(H);
  p.s_in_fp32 = initial_state_dtype == KDA_DTYPE_FP32 ? 1 : 0;
  p.s_out_fp32 = final_state_dtype == KDA_DTYPE_FP32 ? 1 : 0;
  p.s_kv = state_kv;
  p.n_vtiles = static_cast<int32_t>(D / vt);
  p.chunk_rows = chunk;
  p.scale = scale;
  p.lb2 = static_cast<float>(lower_bound * kLog2e);
  p.lam2_floor = needs_decay_floor(lower_bound, chunk) ? static_cast<float>(-kMaxSpan)
                                                       : -INFINITY;
  p.anchor = kda_chunk_anchor(lower_bound, chunk);
  p.ws = workspace;
  p.ws_head_bytes = head_bytes;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const int d = static_cast<int>(D), c = tile_rows(chunk);
  const hipError_t e = split       ? kda::launch_kda_split(p, d, c, vt, hs)
                       : lds_state ? kda::launch_kda_fwd_slds(p, d, c, vt, hs)
                                   : kda::launch_kda_fwd(p, d, c, vt, hs);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_fwd_check(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  float scale, const void* out, const float* A_log, const float* dt_bias,
                  float lower_bound, const void* initial_state, int initial_state_dtype,
                  const void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
                  int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, int chunk_size,
                  int v_tile) {
  int c = 0, vt = 0;
  return resolve(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                 initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                 H, D, chunk_size, v_tile, nullptr, &c, &vt);
}

int kda_fwd_sched(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  float scale, void* out, const float* A_log, const float* dt_bias,
                  float lower_bound, const void* initial_state, int initial_state_dtype,
                  void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
                  int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, void* stream,
                  int chunk_size, int v_tile) {
  return launch(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                H, D, stream, chunk_size, v_tile, nullptr, 0);
}

int kda_fwd_bf16_state(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, float scale, void* out, const float* A_log,
                       const float* dt_bias, float lower_bound, const void* initial_state,
                       int initial_state_dtype, void* final_state, int final_state_dtype,
                       const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                       int64_t H, int64_t D, void* stream, int chunk_size, int v_tile) {
  return launch(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                H, D, stream, chunk_size, v_tile, nullptr, 0, false, nullptr, 0, true);
}

int kda_fwd_ordered(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, float scale, void* out, const float* A_log,
                    const float* dt_bias, float lower_bound, const void* initial_state,
                    int initial_state_dtype, void* final_state, int final_state_dtype,
                    const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H,
                    int64_t D, void* stream, const int32_t* seq_order) {
  if (!seq_order) return KDA_ERR_NULL_ARG;
  return launch(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                H, D, stream, 0, 0, seq_order, 0);
}

int kda_fwd_transposed_state(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, float scale, void* out, const float* A_log,
                             const float* dt_bias, float lower_bound, const void* initial_state,
                             int initial_state_dtype, void* final_state, int final_state_dtype,
                             const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                             int64_t H, int64_t D, void* stream) {
  return launch(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                H, D, stream, 0, 0, nullptr, 1);
}

int kda_longest_first(const int64_t* cu_seqlens, int64_t num_seqs, int32_t* seq_order,
                      void* stream) {
  if (num_seqs < 1 || num_seqs > kda::kMaxOrderSeqs) return KDA_ERR_BAD_VARLEN;
  if (!cu_seqlens || !seq_order) return KDA_ERR_NULL_ARG;
  const Range rc = make_range(cu_seqlens, (num_seqs + 1) * 8);
  const Range ro = make_range(seq_order, num_seqs * 4);
  if (overlaps(rc, ro)) return KDA_ERR_BAD_ALIAS;
  const hipError_t e = kda::launch_longest_first(cu_seqlens, static_cast<int>(num_seqs), seq_order,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
            float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
            const void* initial_state, int initial_state_dtype, void* final_state,
            int final_state_dtype, const int64_t* cu_seqlens, int64_t num_seqs, int64_t B,
            int64_t T, int64_t H, int64_t D, void* stream) {
  return kda_fwd_sched(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                       initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs,
                       B, T, H, D, stream, 0, 0);
}

int64_t kda_split_workspace_bytes(int64_t T_total, int64_t num_seqs, int64_t H, int64_t D,
                                  float lower_bound, int chunk_size) {
  if (T_total < 0 || num_seqs < 1 || H < 1) return KDA_ERR_BAD_SHAPE;
  if (!std::isfinite(lower_bound) || !(lower_bound < 0.f) ||
      !std::isfinite(static_cast<float>(lower_bound * kLog2e)))
    return KDA_ERR_BAD_LOWER_BOUND;
  const int chunk = chunk_size == 0 ? auto_chunk(lower_bound) : chunk_size;
  if (!chunk_rows_valid(chunk)) return KDA_ERR_BAD_SCHEDULE;
  if (!rows_admissible(lower_bound, chunk)) return KDA_ERR_BAD_LOWER_BOUND;
  const int64_t head_bytes = split_head_bytes(T_total, num_seqs, H, D, chunk);
  return head_bytes < 0 ? head_bytes : head_bytes * H;
}

int kda_fwd_split(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  float scale, void* out, const float* A_log, const float* dt_bias,
                  float lower_bound, const void* initial_state, int initial_state_dtype,
                  void* final_state, int final_state_dtype, const int64_t* cu_seqlens,
                  int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t D, void* stream,
                  void* workspace, int64_t workspace_bytes, int chunk_size, int v_tile) {
  return launch(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                H, D, stream, chunk_size, v_tile, nullptr, 0, true, workspace, workspace_bytes);
}

int kda_fwd_split_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float scale, void* out, const float* A_log,
                          const float* dt_bias, float lower_bound, const void* initial_state,
                          int initial_state_dtype, void* final_state, int final_state_dtype,
                          const int64_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                          int64_t H, int64_t D, void* stream, int chunk_size, int v_tile) {
  // the arguments first (nothing touches the device on a validation error), then
  // the workspace size against the scratch array's
  int chunk = 0, vt = 0;
  const int st = resolve(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                         initial_state, initial_state_dtype, final_state, final_state_dtype,
                         cu_seqlens, num_seqs, B, T, H, D, chunk_size, v_tile, nullptr, &chunk,
                         &vt);
  if (st != KDA_OK) return st;
  if (!kda::kda_split_supported(static_cast<int>(D), tile_rows(chunk), vt))
    return KDA_ERR_BAD_SCHEDULE;
  const int64_t head_bytes = split_head_bytes(B * T, num_seqs, H, D, chunk);
  if (head_bytes < 0) return static_cast<int>(head_bytes);
  if (head_bytes > kScratchBytes / H) return KDA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  const int sp = current_scratch(&ws);
  if (sp != KDA_OK) return sp;
  return launch(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                H, D, stream, chunk_size, v_tile, nullptr, 0, true, ws, kScratchBytes);
}

int64_t kda_split_noalloc_max_bytes(void) { return kScratchBytes; }

float kda_chunk_anchor(float lower_bound, int chunk_size) {
  const double span = chunk_span(lower_bound, chunk_size);
  // one-token chunks past the window floor the decay at the window's width
  return static_cast<float>(-0.5 * (chunk_size == 1 && span > kMaxSpan ? kMaxSpan : span));
}

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL_ARG: return "KDA_ERR_NULL_ARG: a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: unsupported sizes";
    case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: unknown state dtype code";
    case KDA_ERR_BAD_VARLEN: return "KDA_ERR_BAD_VARLEN: inconsistent cu_seqlens / num_seqs / B";
    case KDA_ERR_BAD_ALIAS: return "KDA_ERR_BAD_ALIAS: buffers overlap beyond the exact state alias";
    case KDA_ERR_BAD_LOWER_BOUND:
      return "KDA_ERR_BAD_LOWER_BOUND: lower_bound must be finite, negative, above -2.35e38 "
             "and, for a forced chunk of 2 or more tokens, inside its bf16 exponent radius";
    case KDA_ERR_BAD_SCALE: return "KDA_ERR_BAD_SCALE: scale must be finite";
    case KDA_ERR_BAD_SCHEDULE: return "KDA_ERR_BAD_SCHEDULE: unsupported chunk size or value tile";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error";
    case KDA_ERR_BAD_WORKSPACE:
      return "KDA_ERR_BAD_WORKSPACE: the workspace is smaller than kda_split_workspace_bytes";
    case KDA_ERR_SCRATCH_TOO_SMALL:
      return "KDA_ERR_SCRATCH_TOO_SMALL: kda_split_workspace_bytes of this call exceeds the "
             "64 MiB scratch of kda_fwd_split_noalloc (use kda_fwd_split with a workspace)";
    default: return "KDA_ERR_UNKNOWN";
  }
}

}  // extern "C"
