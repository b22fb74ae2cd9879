// Kernel parameter blocks and host-side launchers of the H2O HIP kernels.
// The launchers assume validated arguments (the C-ABI layer checks them).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace h2o {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

// Prefill block numbering. MI355X hands workgroups to its 8 XCDs round-robin by block
// index, and each XCD has its own L2. A unit (sequence, head) has `per_unit` blocks that
// read the same K/V (or Q) rows, so a unit's blocks all go to XCD unit % 8. Each XCD takes
// its units in groups of about one resident round (~64 workgroups: 32 CUs x 2) and issues
// a group's blocks block-index-major, so the longest blocks of the group start first (r = 0
// is the longest) while the group's blocks share L2. Units are padded to whole groups;
// blocks of padding units exit at once.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_group_units(int64_t units, int per_unit) {
  const int64_t per_xcd = (units + kXcds - 1) / kXcds;
  int64_t g = (64 + per_unit - 1) / per_unit;
  if (g > per_xcd) g = per_xcd;
  return g < 1 ? 1 : (int)g;
}
inline int64_t xcd_grid_blocks(int64_t units, int per_unit) {
  const int64_t g = xcd_group_units(units, per_unit);
  const int64_t groups = (units + kXcds * g - 1) / (kXcds * g);
  return groups * kXcds * g * per_unit;
}
// Inverse of that numbering: block `bid` works on block `r` of unit `unit`; unit >= units
// marks a padding block.
struct UnitBlock { int unit, r; };
__device__ __forceinline__ UnitBlock xcd_unit_block(int bid, int units, int per_unit) {
  const int g = xcd_group_units(units, per_unit);
  const int x = bid & 7, j = bid >> 3;
  const int grp = j / (g * per_unit), w = j - grp * (g * per_unit);
  const int r = w / g;
  return {(grp * g + (w - r * g)) * 8 + x, r};
}

struct DecodeParams {
  const void* q;        // [units][D]
  const void* k_new;    // [units][D]
  const void* v_new;    // [units][D]
  void* k_slots;        // [units][k][D]
  void* v_slots;        // [units][k][D]
  int32_t* slot_pos;    // [units][k]
  float* acc;           // [units][k]
  float* out;           // [units][D] fp32
  int32_t* victim_slot; // [units] or null
  int32_t* evicted_pos; // [units] or null
  float* evicted_acc;   // [units] or null
  const int32_t* tpos;  // [batch] per-sequence positions (device), or null: t for all
  int32_t policy;       // eviction ranking, h2o_policy
  int32_t policy_param;
  int32_t units;
  int32_t heads;        // units of one sequence
  int32_t k;
  int32_t k_local;
  int32_t t;
  float qk_scale;       // log2(e) / sqrt(D) (times k_scale for E4M3 slots): log2-domain logits
  float k_inv, v_inv;   // E4M3 slots: fl32(1 / k_scale), fl32(1 / v_scale)
  float v_scale;        // E4M3 slots: the output is scaled by it once
};

// Eviction rankings (the C ABI's h2o_policy). The fp32 value a candidate is ranked by:
// the running score (H2O), this step's probability (Top-K), or a 0/1 position class
// (sinks: 1 below policy_param; strided: 1 on multiples of policy_param). All are >= 0, so
// their bit patterns order like the values.
enum : int { kPolicyH2O = 0, kPolicySinks = 1, kPolicyStrided = 2, kPolicyTopK = 3 };
__host__ __device__ inline float policy_key(int policy, int param, float acc, float p, int pos) {
  if (policy == kPolicyH2O) return acc;
  if (policy == kPolicyTopK) return p;
  if (policy == kPolicySinks) return pos < param ? 1.f : 0.f;
  return pos % param == 0 ? 1.f : 0.f;
}
// The seed score of prompt position j: c is the column sum under H2O and the prompt's last
// attention row P[T-1][j] under Top-K (the highest current attention); position policies
// rank by their 0/1 class.
__host__ __device__ inline float policy_seed(int policy, int param, float c, int j) {
  if (policy == kPolicySinks) return j < param ? 1.f : 0.f;
  if (policy == kPolicyStrided) return j % param == 0 ? 1.f : 0.f;
  return c;
}

// A unit's own bound from a per-sequence device array (clamped to [0, hi], so a bad entry
// cannot address outside the buffers), or the shared value when there is no array.
__device__ __forceinline__ int unit_bound(const int32_t* per_seq, int unit, int heads, int shared,
                                          int hi) {
  if (!per_seq) return shared;
  const int v = per_seq[unit / heads];
  return v < 0 ? 0 : (v > hi ? hi : v);
}

// Column-sum partials. The prefill leaves, per unit, one partial row per block of `pb`
// query rows: row r holds, for each key j < min(T, (r + 1) * pb), the sum of P_ij over the
// block's rows i, and starts at pb * r * (r + 1) / 2 within the unit's stretch. The seed
// adds the rows that cover key j in row order.
__host__ __device__ inline int64_t colpart_row_offset(int64_t r, int pb) {
  return (int64_t)pb * r * (r + 1) / 2;
}
__host__ __device__ inline int64_t colpart_stride(int64_t T, int pb) {
  const int64_t rows = (T + pb - 1) / pb;
  return rows > 0 ? colpart_row_offset(rows - 1, pb) + T : 0;
}
// Query rows per partial row of the MFMA prefill (its attention workgroup's block).
constexpr int kPrefillPartRows = 128;

struct PrefillParams {
  const void* q;        // [units][T][D]
  const void* k;
  const void* v;
  float* out;           // [units][T][D]
  float* lse2;          // [units][T] row log-sum-exp, log2 domain (fp32 path only)
  float* colpart;       // [units][colpart_stride(T, part_rows)] column-sum partials
  const int32_t* lens;  // [batch] per-sequence prompt lengths <= T (device), or null: T
  int32_t units;
  int32_t heads;        // units of one sequence
  int32_t T;            // rows stored per unit (the stride of q, k, v, out)
  float qk_scale;       // log2(e) / sqrt(D)
};

struct SeedParams {
  const void* k;        // prompt K/V [units][T][D]
  const void* v;
  const float* colpart; // [units][colpart_stride(T, part_rows)]
  float* colsum;        // [units][T]: the summed column sums are written here
  const float* rank;    // [units][T] seed scores other than the column sums (Top-K: the last
                        // prompt row's attention), or null
  const int32_t* lens;  // [batch] per-sequence prompt lengths <= T (device), or null: T
  void* k_slots;
  void* v_slots;
  int32_t* slot_pos;
  float* acc;
  int32_t units;
  int32_t heads;        // units of one sequence
  int32_t T;            // rows stored per unit
  int32_t part_rows;    // query rows per partial row
  int32_t k_heavy;
  int32_t k_local;
  int32_t policy;       // seeding ranking, h2o_policy
  int32_t policy_param;
  float k_inv, v_inv;   // E4M3 slots: fl32(1 / k_scale), fl32(1 / v_scale)
};

// The prompt's last attention row, P[T-1][j] for j < T (fp32), per unit: the Top-K seed
// scores.
struct LastRowParams {
  const void* q;        // prompt Q/K [units][T][D]
  const void* k;
  float* rank;          // [units][T]
  const int32_t* lens;  // [batch] per-sequence prompt lengths <= T (device), or null: T
  int32_t units;
  int32_t heads;
  int32_t T;            // rows stored per unit
  int32_t k_slots;      // k: a unit whose prompt fits (T <= k) needs no ranking
  float qk_scale;       // log2(e) / sqrt(D)
};

struct ResetParams {
  int32_t* slot_pos;
  float* acc;
  int64_t n;            // units * k
};

// Decode launch plan: splits == 0 -> one resident workgroup of `threads` threads per
// unit; splits > 0 -> a partial kernel with `splits` workgroups per unit, then a
// combine kernel with one workgroup per unit.
struct DecodePlan {
  int threads;
  int splits;
};
DecodePlan plan_decode(int elem_bytes, int D, int k, int units);
constexpr int kMaxSplits = 160;   // enough for k <= 8192 at 56 slots per split (147)

// Workspace of the split decode: per-split partials plus the step's logits.
struct SplitScratch {
  float* part_ml;       // [units][splits][2]  (max, sum) in the log2 domain
  float* part_o;        // [units][splits][D]  unnormalised output
  float* logits;        // [units][k + 1]
  int splits;
};
size_t decode_scratch_bytes(int elem_bytes, int D, int k, int units);
SplitScratch carve_decode_scratch(int elem_bytes, int D, int k, int units, void* scratch);

hipError_t launch_reset(const ResetParams& p, hipStream_t s);
// f8: the slots hold E4M3 codes (fp16 / bf16 inputs only).
hipError_t launch_decode(DType dt, bool f8, int D, const DecodeParams& p, const SplitScratch& w,
                         hipStream_t s);
// fp16 / bf16 storage: MFMA kernels.
hipError_t launch_prefill_attn_mfma(DType dt, int D, const PrefillParams& p, hipStream_t s);
// fp32 storage: vector-ALU kernels.
hipError_t launch_prefill_attn_f32(int D, const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_colsum_f32(int D, const PrefillParams& p, hipStream_t s);
hipError_t launch_seed(DType dt, bool f8, int D, const SeedParams& p, hipStream_t s);
hipError_t launch_last_row(DType dt, int D, const LastRowParams& p, hipStream_t s);

}  // namespace h2o
