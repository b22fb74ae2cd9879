// C ABI of the H2O hot path (declared in include/h2o.h): argument checks,
// dtype / head_dim dispatch, workspace carving and kernel enqueue.
//
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing, touches no memory and needs no device (the checks are
// exercised without a GPU). No call allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/h2o.h"
#include "h2o_kernels.hpp"

namespace {

thread_local char g_err[512] = "";

h2o_status fail(h2o_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

h2o_status hip_fail(hipError_t e, const char* what) {
  return fail(H2O_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(int32_t dt) { return dt == H2O_F32 ? 4 : 2; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr size_t kWsAlign = 256;

h2o_status check_desc(const h2o_cache_desc* c) {
  if (!c) return fail(H2O_ERR_INVALID, "cache descriptor is NULL");
  if (c->batch < 1 || c->heads < 1)
    return fail(H2O_ERR_INVALID, "batch (%d) and heads (%d) must be >= 1", c->batch, c->heads);
  if (c->dtype != H2O_F32 && c->dtype != H2O_F16 && c->dtype != H2O_BF16)
    return fail(H2O_ERR_INVALID, "dtype %d is not an h2o_dtype", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(H2O_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (c->k_heavy < 0) return fail(H2O_ERR_INVALID, "k_heavy %d < 0", c->k_heavy);
  if (c->k_local < 1)
    return fail(H2O_ERR_INVALID, "k_local %d < 1: the new token must stay in the recent window",
                c->k_local);
  if (c->policy < H2O_POLICY_H2O || c->policy > H2O_POLICY_TOPK)
    return fail(H2O_ERR_INVALID, "policy %d is not an h2o_policy", c->policy);
  if ((c->policy == H2O_POLICY_SINKS && c->policy_param < 0) ||
      (c->policy == H2O_POLICY_STRIDED && c->policy_param < 1))
    return fail(H2O_ERR_INVALID, "policy_param %d out of range for policy %d", c->policy_param,
                c->policy);
  if (c->slot_format != H2O_SLOTS_INPUT && c->slot_format != H2O_SLOTS_FP8_E4M3)
    return fail(H2O_ERR_INVALID, "slot_format %d is not an h2o_slot_format", c->slot_format);
  if (c->slot_format == H2O_SLOTS_FP8_E4M3) {
    if (c->dtype == H2O_F32)
      return fail(H2O_ERR_UNSUPPORTED, "E4M3 slots take fp16 or bf16 inputs, not fp32");
    if (!(std::isfinite(c->k_scale) && c->k_scale > 0.f && std::isfinite(c->v_scale) &&
          c->v_scale > 0.f))
      return fail(H2O_ERR_INVALID, "E4M3 scales must be finite and > 0 (k_scale %g, v_scale %g)",
                  (double)c->k_scale, (double)c->v_scale);
  }
  if ((int64_t)c->k_heavy + c->k_local > H2O_MAX_SLOTS)
    return fail(H2O_ERR_UNSUPPORTED, "k = %lld exceeds H2O_MAX_SLOTS (%d)",
                (long long)c->k_heavy + c->k_local, H2O_MAX_SLOTS);
  if ((int64_t)c->batch * c->heads > 0x7fffffffLL)
    return fail(H2O_ERR_UNSUPPORTED, "batch * heads exceeds 2^31 - 1");
  if (!c->k_slots || !c->v_slots || !c->slot_pos || !c->acc_score)
    return fail(H2O_ERR_INVALID, "a cache array pointer is NULL");
  if (!aligned(c->k_slots, 16) || !aligned(c->v_slots, 16))
    return fail(H2O_ERR_INVALID, "k_slots / v_slots must be 16-byte aligned");
  if (!aligned(c->slot_pos, 4) || !aligned(c->acc_score, 4))
    return fail(H2O_ERR_INVALID, "slot_pos / acc_score must be 4-byte aligned");
  return H2O_OK;
}

int units_of(const h2o_cache_desc* c) { return c->batch * c->heads; }
int slots_of(const h2o_cache_desc* c) { return c->k_heavy + c->k_local; }

// Workspace: scratch shared by prefill (column-sum partial rows and the column sums; the
// fp32 path also keeps each row's log-sum-exp) and the split decode (per-split partials and
// logits); its contents on entry never matter.
int part_rows_of(const h2o_cache_desc* c, int64_t T) {
  return c->dtype == H2O_F32 ? (int)(T > 0 ? T : 1) : h2o::kPrefillPartRows;
}
struct PrefillLayout {
  size_t lse2, colpart, colsum, rank, total;   // byte offsets of the parts, total size
};
// Top-K seeds by the last prompt row's attention, kept in its own [units][T] part.
PrefillLayout prefill_layout(const h2o_cache_desc* c, int64_t T) {
  const size_t units = (size_t)units_of(c);
  const size_t rows = round_up(units * (size_t)T * sizeof(float), kWsAlign);
  const size_t part = round_up(
      units * (size_t)h2o::colpart_stride(T, part_rows_of(c, T)) * sizeof(float), kWsAlign);
  PrefillLayout l{};
  l.lse2 = 0;
  l.colpart = c->dtype == H2O_F32 ? rows : 0;
  l.colsum = l.colpart + part;
  l.rank = l.colsum + rows;
  l.total = l.rank + (c->policy == H2O_POLICY_TOPK ? rows : 0);
  return l;
}
size_t prefill_scratch(const h2o_cache_desc* c, int64_t T) { return prefill_layout(c, T).total; }

size_t decode_scratch(const h2o_cache_desc* c) {
  return h2o::decode_scratch_bytes((int)elem_bytes(c->dtype), c->head_dim, slots_of(c),
                                   units_of(c));
}

h2o::DType dtype_of(const h2o_cache_desc* c) { return static_cast<h2o::DType>(c->dtype); }
bool f8_of(const h2o_cache_desc* c) { return c->slot_format == H2O_SLOTS_FP8_E4M3; }
// fl32(1 / scale) of an E4M3 slot format (unused otherwise).
float inv_of(const h2o_cache_desc* c, float scale) { return f8_of(c) ? 1.0f / scale : 1.0f; }

float qk_scale(int d) { return (float)(1.4426950408889634 / std::sqrt((double)d)); }

// Scratch of h2o_decode_step_noalloc: a file-scope device array (each GPU the library runs
// on holds its own copy until the process ends). Host code uses the array's device address
// from hipGetSymbolAddress, taken once per device with that device current; the array's
// name in host code is only a host-side stand-in.
static __device__ __align__(256) unsigned char scratch[H2O_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch; the stream must belong to that
// device.
h2o_status noalloc_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return hip_fail(e, "hipGetDevice");
  if (stream) {
    int sdev = -1;
    if (hipError_t e = hipStreamGetDevice(stream, &sdev)) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(H2O_ERR_INVALID, "the stream belongs to device %d but device %d is current",
                  sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(H2O_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return H2O_OK;
}

}  // namespace

extern "C" {

const char* h2o_status_str(h2o_status s) {
  switch (s) {
    case H2O_OK: return "H2O_OK";
    case H2O_ERR_INVALID: return "H2O_ERR_INVALID";
    case H2O_ERR_UNSUPPORTED: return "H2O_ERR_UNSUPPORTED";
    case H2O_ERR_WORKSPACE: return "H2O_ERR_WORKSPACE";
    case H2O_ERR_HIP: return "H2O_ERR_HIP";
  }
  return "H2O_ERR_UNKNOWN";
}

const char* h2o_last_error(void) { return g_err; }

size_t h2o_workspace_bytes(const h2o_cache_desc* c, int32_t max_prompt) {
  if (check_desc(c) != H2O_OK || max_prompt < 0) return 0;
  const size_t a = prefill_scratch(c, max_prompt), b = decode_scratch(c);
  return a > b ? a : b;
}

h2o_status h2o_reset(const h2o_cache_desc* c, void* stream) {
  g_err[0] = 0;
  if (h2o_status st = check_desc(c)) return st;
  h2o::ResetParams p{c->slot_pos, c->acc_score,
                     (int64_t)c->batch * c->heads * (c->k_heavy + c->k_local)};
  if (hipError_t e = h2o::launch_reset(p, static_cast<hipStream_t>(stream)))
    return hip_fail(e, "reset launch");
  return H2O_OK;
}

}  // extern "C"

namespace {

// The prefill behind both entry points; lens = NULL means every sequence has length T.
h2o_status prefill_impl(const h2o_cache_desc* c, const void* q, const void* k, const void* v,
                        int32_t T, const int32_t* lens, float* out, float* colsum_out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (h2o_status st = check_desc(c)) return st;
  if (T < 0) return fail(H2O_ERR_INVALID, "prompt length T = %d < 0", T);
  if (!q || !k || !v || !out) return fail(H2O_ERR_INVALID, "q, k, v and out must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(H2O_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
  if (colsum_out && !aligned(colsum_out, 4))
    return fail(H2O_ERR_INVALID, "colsum_out must be 4-byte aligned");
  const int64_t units = (int64_t)c->batch * c->heads;
  if (h2o::xcd_grid_blocks(units, ((int64_t)T + 15) / 16) > 0x7fffffffLL)
    return fail(H2O_ERR_UNSUPPORTED, "batch * heads * ceil(T / 16) exceeds the grid limit");
  // The attention kernels address one unit's K/V rows through a buffer descriptor whose
  // byte range is a signed 32-bit count.
  if ((int64_t)T * c->head_dim * (int64_t)elem_bytes(c->dtype) > 0x7fffffffLL)
    return fail(H2O_ERR_UNSUPPORTED, "T * head_dim * element size exceeds 2^31 - 1 bytes");
  const size_t need = prefill_scratch(c, T);
  if (T > 0 && (!workspace || workspace_bytes < need))
    return fail(H2O_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  if (workspace && !aligned(workspace, kWsAlign))
    return fail(H2O_ERR_INVALID, "workspace must be %zu-byte aligned", kWsAlign);
  if (T == 0) return H2O_OK;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const PrefillLayout lay = prefill_layout(c, T);
  float* lse2 = reinterpret_cast<float*>(ws + lay.lse2);
  float* colpart = reinterpret_cast<float*>(ws + lay.colpart);
  float* colsum = colsum_out ? colsum_out : reinterpret_cast<float*>(ws + lay.colsum);
  const int D = c->head_dim;
  const h2o::DType dt = dtype_of(c);

  h2o::PrefillParams pp{q, k, v, out, lse2, colpart, lens, (int32_t)units, c->heads, T,
                        qk_scale(D)};
  hipError_t e;
  if (dt == h2o::DType::F32) {
    if ((e = h2o::launch_prefill_attn_f32(D, pp, s))) return hip_fail(e, "prefill attention launch");
    if ((e = h2o::launch_prefill_colsum_f32(D, pp, s))) return hip_fail(e, "prefill colsum launch");
  } else {
    if ((e = h2o::launch_prefill_attn_mfma(dt, D, pp, s)))
      return hip_fail(e, "prefill attention launch");
  }
  float* rank = nullptr;
  if (c->policy == H2O_POLICY_TOPK) {
    rank = reinterpret_cast<float*>(ws + lay.rank);
    h2o::LastRowParams lp{q, k, rank, lens, (int32_t)units, c->heads, T, slots_of(c),
                          qk_scale(D)};
    if ((e = h2o::launch_last_row(dt, D, lp, s))) return hip_fail(e, "last-row launch");
  }
  h2o::SeedParams sp{k, v, colpart, colsum, rank, lens, c->k_slots, c->v_slots, c->slot_pos,
                     c->acc_score, (int32_t)units, c->heads, T, part_rows_of(c, T), c->k_heavy,
                     c->k_local, c->policy, c->policy_param, inv_of(c, c->k_scale),
                     inv_of(c, c->v_scale)};
  if ((e = h2o::launch_seed(dt, f8_of(c), D, sp, s))) return hip_fail(e, "seed launch");
  return H2O_OK;
}

// The decode step behind the entry points; tpos = NULL means every sequence is at t.
// noalloc: the scratch is the library's static array instead of the caller's workspace.
h2o_status decode_impl(const h2o_cache_desc* c, int64_t t, const int32_t* tpos, const void* q,
                       const void* k_new, const void* v_new, float* out,
                       const h2o_decode_aux* aux, void* workspace, size_t workspace_bytes,
                       void* stream, bool noalloc = false) {
  g_err[0] = 0;
  if (h2o_status st = check_desc(c)) return st;
  if (t < 0 || t >= (int64_t)H2O_MAX_POSITION)
    return fail(H2O_ERR_INVALID, "position t = %lld outside [0, 2^31 - 1)", (long long)t);
  if (!q || !k_new || !v_new || !out)
    return fail(H2O_ERR_INVALID, "q, k_new, v_new and out must not be NULL");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16))
    return fail(H2O_ERR_INVALID, "q, k_new, v_new and out must be 16-byte aligned");
  if (aux && ((aux->victim_slot && !aligned(aux->victim_slot, 4)) ||
              (aux->evicted_pos && !aligned(aux->evicted_pos, 4)) ||
              (aux->evicted_acc && !aligned(aux->evicted_acc, 4))))
    return fail(H2O_ERR_INVALID, "aux arrays must be 4-byte aligned");

  const h2o::DecodePlan plan =
      h2o::plan_decode((int)elem_bytes(c->dtype), c->head_dim, slots_of(c), units_of(c));
  if (plan.splits > h2o::kMaxSplits)
    return fail(H2O_ERR_UNSUPPORTED, "k = %d needs %d decode splits, more than %d",
                slots_of(c), plan.splits, h2o::kMaxSplits);
  if ((int64_t)units_of(c) * (plan.splits ? plan.splits : 1) > 0x7fffffffLL)
    return fail(H2O_ERR_UNSUPPORTED, "batch * heads * %d decode workgroups exceed the grid limit",
                plan.splits);
  const size_t scratch = decode_scratch(c);
  if (noalloc) {
    if (scratch > (size_t)H2O_NOALLOC_SCRATCH_BYTES)
      return fail(H2O_ERR_UNSUPPORTED,
                  "this shape needs %zu bytes of decode scratch; the static scratch of the "
                  "allocation-free entry point holds %zu",
                  scratch, (size_t)H2O_NOALLOC_SCRATCH_BYTES);
  } else {
    if (scratch > 0 && (!workspace || workspace_bytes < scratch))
      return fail(H2O_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? workspace_bytes : (size_t)0, scratch);
    if (workspace && !aligned(workspace, kWsAlign))
      return fail(H2O_ERR_INVALID, "workspace must be %zu-byte aligned", kWsAlign);
  }
  // Every argument is checked; only now does the allocation-free path ask for its scratch.
  if (noalloc && scratch > 0)
    if (h2o_status st = noalloc_scratch(&workspace, static_cast<hipStream_t>(stream))) return st;

  const int D = c->head_dim;
  const int32_t kk = c->k_heavy + c->k_local;
  const h2o::SplitScratch w =
      scratch ? h2o::carve_decode_scratch((int)elem_bytes(c->dtype), D, kk, units_of(c), workspace)
              : h2o::SplitScratch{};
  h2o::DecodeParams p{q, k_new, v_new, c->k_slots, c->v_slots, c->slot_pos, c->acc_score, out,
                      aux ? aux->victim_slot : nullptr, aux ? aux->evicted_pos : nullptr,
                      aux ? aux->evicted_acc : nullptr, tpos, c->policy, c->policy_param,
                      (int32_t)(c->batch * c->heads),
                      c->heads, kk, c->k_local, (int32_t)t,
                      f8_of(c) ? qk_scale(D) * c->k_scale : qk_scale(D), inv_of(c, c->k_scale),
                      inv_of(c, c->v_scale), f8_of(c) ? c->v_scale : 1.0f};
  if (hipError_t e = h2o::launch_decode(dtype_of(c), f8_of(c), D, p, w,
                                        static_cast<hipStream_t>(stream)))
    return hip_fail(e, "decode launch");
  return H2O_OK;
}

}  // namespace

extern "C" {

h2o_status h2o_prefill(const h2o_cache_desc* c, const void* q, const void* k, const void* v,
                       int32_t T, float* out, float* colsum_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return prefill_impl(c, q, k, v, T, nullptr, out, colsum_out, workspace, workspace_bytes,
                      stream);
}

h2o_status h2o_prefill_ragged(const h2o_cache_desc* c, const void* q, const void* k,
                              const void* v, int32_t T_max, const int32_t* lens, float* out,
                              float* colsum_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  g_err[0] = 0;
  if (!lens || !aligned(lens, 4))
    return fail(H2O_ERR_INVALID, "lens must be a non-NULL, 4-byte aligned device array");
  return prefill_impl(c, q, k, v, T_max, lens, out, colsum_out, workspace, workspace_bytes,
                      stream);
}

h2o_status h2o_decode_step(const h2o_cache_desc* c, int64_t t, const void* q, const void* k_new,
                           const void* v_new, float* out, const h2o_decode_aux* aux,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(c, t, nullptr, q, k_new, v_new, out, aux, workspace, workspace_bytes,
                     stream);
}

h2o_status h2o_decode_step_noalloc(const h2o_cache_desc* c, int64_t t, const void* q,
                                   const void* k_new, const void* v_new, float* out,
                                   const h2o_decode_aux* aux, void* stream) {
  return decode_impl(c, t, nullptr, q, k_new, v_new, out, aux, nullptr, 0, stream, true);
}

h2o_status h2o_decode_step_ragged(const h2o_cache_desc* c, const int32_t* t, const void* q,
                                  const void* k_new, const void* v_new, float* out,
                                  const h2o_decode_aux* aux, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!t || !aligned(t, 4))
    return fail(H2O_ERR_INVALID, "t must be a non-NULL, 4-byte aligned device array");
  return decode_impl(c, 0, t, q, k_new, v_new, out, aux, workspace, workspace_bytes, stream);
}

}  // extern "C"
