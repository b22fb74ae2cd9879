/*
 * h2o.h - C ABI of the H2O (Heavy-Hitter Oracle) KV-cache eviction hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   - H2O blog, ttsmallhot.github.io/posts/8adb0d1a: §2.1.1 (attention is the
 *     row softmax of Q K^T / sqrt(d)), §2.1.2 (a token's accumulated attention
 *     score), §2.2 (a budget of k slots split into k_local recent tokens and
 *     k_heavy heavy hitters; a running score per token; greedy eviction of the
 *     lowest score outside the recent tokens), §2.3 (the evicted slot is marked
 *     free and the new token's K/V is written at that address, no compaction).
 *   - "H2O Heavy-Hitter Oracle 分析" (liuhc.cn): §3.1 (heavy hitters = top-k of
 *     the cumulative attention per head), §3.2 (victim = argmin of the score;
 *     the new token always joins the cache).
 *
 * Units. One unit is one (sequence, head) of one layer. Units are independent;
 * each has its own k = k_heavy + k_local slots. A layer's cache is described by
 * an h2o_cache_desc; several layers use several descriptors.
 *
 * Memory. Every pointer passed to these functions is DEVICE memory owned by the
 * caller (except the descriptor and aux structs themselves, which are host
 * structs read during the call only). The library never allocates, frees or
 * synchronises, keeps no pointer after a call returns, and holds no state.
 *
 * Streams. `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * Every call enqueues its kernels on that stream and returns without waiting.
 * Calls on one descriptor must be ordered on one stream; calls on distinct
 * descriptors may run concurrently.
 *
 * Errors. Every argument is checked on the host before anything is enqueued;
 * on a failed check the call returns a non-zero status, enqueues nothing and
 * changes nothing, and h2o_last_error() describes the failure. A launch error
 * reported by the HIP runtime maps to H2O_ERR_HIP. Faults inside a kernel
 * surface at the caller's next synchronisation. No C++ exception crosses this
 * interface. Misuse that cannot be checked (decode positions out of order,
 * buffers that are too small) is undefined behaviour.
 *
 * Numerics. Q/K/V are stored in `dtype`, the K/V slots in `dtype` or, on
 * request, as FP8 E4M3 codes (h2o_slot_format below); all arithmetic is
 * fp32. Attention outputs are written as fp32. Scores (acc_score) are fp32:
 * prefill seeds a slot with its fp32 column sum, each decode step adds the
 * token's fp32 probability with one fp32 add. Eviction decisions are taken on
 * those fp32 scores, ties broken towards the older position.
 */
#ifndef H2O_H_
#define H2O_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  H2O_OK = 0,
  H2O_ERR_INVALID = 1,      /* a null/misaligned pointer or an out-of-range value */
  H2O_ERR_UNSUPPORTED = 2,  /* a valid request this build does not implement */
  H2O_ERR_WORKSPACE = 3,    /* workspace missing or smaller than h2o_workspace_bytes */
  H2O_ERR_HIP = 4           /* the HIP runtime reported an error */
} h2o_status;

typedef enum { H2O_F32 = 0, H2O_F16 = 1, H2O_BF16 = 2 } h2o_dtype;

/*
 * Eviction ranking. Seeding keeps the last k_local prompt positions plus the
 * k_heavy others ranked highest by (seed score, position); a decode step with a
 * full cache evicts, among slots with slot_pos <= t - k_local, the smallest
 * (key, slot_pos), compared lexicographically.
 *   H2O_POLICY_H2O      seed score: column sum c_j; key: acc_score (H2O blog
 *                       §2.2; analysis page §3.1, §3.2)
 *   H2O_POLICY_SINKS    seed score: 1 for positions < policy_param, else 0; key
 *                       likewise: the first policy_param tokens stay (with
 *                       k_heavy = policy_param the cache is those sinks plus the
 *                       most recent window, the StreamLLM comparison of the blog
 *                       §3.3 Q1); policy_param >= 0
 *   H2O_POLICY_STRIDED  seed score and key: 1 for positions that are multiples
 *                       of policy_param, else 0 (blog §3.1.1 "Strided"):
 *                       the window plus the latest multiples; policy_param >= 1
 *   H2O_POLICY_TOPK     seed score: the prompt's last attention row,
 *                       P[T-1][j]; key: the slot's attention probability in
 *                       this step (blog §3.1.1 "Top-K": the tokens with the
 *                       highest current attention stay, the token attended
 *                       least now leaves)
 * acc_score accumulates every step under every policy. Local is H2O with
 * k_heavy = 0; heavy-only is k_local = 1.
 */
typedef enum {
  H2O_POLICY_H2O = 0,
  H2O_POLICY_SINKS = 1,
  H2O_POLICY_STRIDED = 2,
  H2O_POLICY_TOPK = 3
} h2o_policy;

/*
 * Slot storage. The H2O blog (§3.3 Q3) reports that H2O combines with KV
 * quantisation and names no scheme; this build offers OCP FP8 E4M3 slots:
 *   H2O_SLOTS_INPUT     k_slots / v_slots hold K/V in dtype (the default)
 *   H2O_SLOTS_FP8_E4M3  they hold E4M3 codes, one byte per element (1 sign,
 *                       4 exponent bits with bias 7, 3 mantissa bits; largest
 *                       finite value 448). A K row x enters a slot as codes
 *                       e4m3(fl32(x * fl32(1 / k_scale))), rounded to nearest
 *                       with ties to even and saturated at +-448, and is read
 *                       back as code value * k_scale (V likewise with v_scale).
 *                       The new token's K/V are quantised before the step's
 *                       attention reads them, so a step attends to exactly
 *                       what the cache holds afterwards; prefill attention
 *                       reads the prompt's own K/V. dtype must be H2O_F16 or
 *                       H2O_BF16 (H2O_ERR_UNSUPPORTED for H2O_F32); k_scale
 *                       and v_scale must be finite and > 0.
 */
typedef enum { H2O_SLOTS_INPUT = 0, H2O_SLOTS_FP8_E4M3 = 1 } h2o_slot_format;

/* Limits of this build. */
#define H2O_MAX_SLOTS 8192        /* k = k_heavy + k_local */
#define H2O_MAX_POSITION 0x7fffffff

/*
 * One layer's cache. All arrays are device memory, caller-owned, contiguous,
 * indexed [batch][heads][k] (slot arrays) or [batch][heads][k][head_dim] (rows).
 *   batch, heads  >= 1
 *   head_dim      64 or 128
 *   k_heavy       >= 0 ; k_local >= 1 ; 1 <= k_heavy + k_local <= H2O_MAX_SLOTS
 *                 (k_local >= 1 keeps the new token out of the candidates:
 *                 the recent window is positions (t - k_local, t])
 *   dtype         storage type of Q/K/V, and of k_slots/v_slots unless
 *                 slot_format says otherwise (h2o_dtype)
 *   k_slots, v_slots  16-byte aligned; [batch][heads][k][head_dim] elements of
 *                 dtype, or of one byte with H2O_SLOTS_FP8_E4M3
 *   slot_pos      int32 absolute position held by each slot, -1 = free
 *   acc_score     fp32 accumulated attention score of each slot
 *   policy, policy_param  eviction ranking (h2o_policy above); 0, 0 is H2O
 *   slot_format   h2o_slot_format; 0 stores the slots in dtype
 *   k_scale, v_scale  E4M3 scales (read only with H2O_SLOTS_FP8_E4M3)
 * Valid slots always form a prefix [0, n_valid) of each unit's slots.
 */
typedef struct {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t k_heavy;
  int32_t k_local;
  int32_t dtype;
  void* k_slots;
  void* v_slots;
  int32_t* slot_pos;
  float* acc_score;
  int32_t policy;
  int32_t policy_param;
  int32_t slot_format;
  float k_scale;
  float v_scale;
} h2o_cache_desc;

/*
 * Optional per-step record of the decode decision, each array [batch][heads]
 * int32/fp32 device memory, 4-byte aligned; any pointer may be NULL.
 *   victim_slot  slot that was overwritten, or -1 when the token was appended
 *                to a free slot (nothing evicted)
 *   evicted_pos  position that was evicted, or -1
 *   evicted_acc  its final score (after this step's add), or 0
 */
typedef struct {
  int32_t* victim_slot;
  int32_t* evicted_pos;
  float* evicted_acc;
} h2o_decode_aux;

/*
 * h2o_reset - mark every slot free: slot_pos = -1, acc_score = 0.
 * The slot rows are left as they are. (H2O blog §2.3: a free slot is only
 * marked, never cleared or compacted.)
 */
h2o_status h2o_reset(const h2o_cache_desc* cache, void* stream);

/*
 * h2o_workspace_bytes - device workspace needed by h2o_prefill with prompts of
 * up to max_prompt tokens and by h2o_decode_step on this descriptor's shape.
 * Returns 0 for an invalid descriptor or max_prompt < 0.
 *
 * Workspace contract: 256-byte aligned device memory owned by the caller. It is
 * scratch: its contents on entry are ignored and on return are unspecified
 * (prefill keeps per-query-block partial column sums there, about T^2 / 256
 * floats per unit for fp16/bf16, the column sums when colsum_out is NULL, and
 * under H2O_POLICY_TOPK the last prompt row's attention, T floats per unit;
 * a decode that spreads a unit's slots over several workgroups keeps
 * per-workgroup partials there). The size grows with max_prompt, so a
 * workspace sized for max_prompt serves every shorter prompt. One workspace
 * must not be used by two calls that can run at the same time.
 */
size_t h2o_workspace_bytes(const h2o_cache_desc* cache, int32_t max_prompt);

/*
 * h2o_prefill - causal attention over a prompt of T tokens, its softmax column
 * sums, and the seeding of each unit's cache.
 *   q, k, v     [batch][heads][T][head_dim] in dtype, 16-byte aligned
 *   T           0 <= T <= H2O_MAX_POSITION; T = 0 enqueues nothing
 *   out         [batch][heads][T][head_dim] fp32, 16-byte aligned:
 *               out_i = sum_{j<=i} P_ij v_j, P = causal row softmax of
 *               q k^T / sqrt(head_dim) (H2O blog §2.1.1)
 *   colsum_out  NULL or [batch][heads][T] fp32: c_j = sum_{i>=j} P_ij, the
 *               cumulative attention of each prompt token (analysis page §3.1)
 *   workspace   at least h2o_workspace_bytes(cache, T) bytes (see the workspace
 *               contract above)
 * Seeding (H2O blog §2.2; analysis page §3.1): if T <= k every position is
 * kept; otherwise the last k_local positions plus the k_heavy positions of
 * [0, T - k_local) with the highest fp32 seed score (c_j under H2O; see
 * h2o_policy for the others; ties: the newer position ranks higher) are kept. Kept positions fill slots 0.. in ascending position order
 * (K/V rows copied from k and v, slot_pos = position, acc_score = fp32 c_j);
 * every other slot is marked free. All previous slot contents are replaced.
 * Returns H2O_ERR_UNSUPPORTED when one unit's prompt rows exceed 2^31 - 1 bytes
 * (T * head_dim * element size) or the launch grid would exceed 2^31 - 1
 * workgroups; nothing is enqueued then.
 */
h2o_status h2o_prefill(const h2o_cache_desc* cache, const void* q, const void* k,
                       const void* v, int32_t T, float* out, float* colsum_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * h2o_decode_step - one generated token per unit, at position t.
 *   t           number of tokens the sequence held before this one,
 *               0 <= t < H2O_MAX_POSITION; successive calls on a descriptor
 *               must pass t = T, T + 1, ... (T = the prompt length)
 *   q, k_new, v_new  [batch][heads][head_dim] in dtype, 16-byte aligned
 *   out         [batch][heads][head_dim] fp32, 16-byte aligned
 *   aux         NULL or a host struct of optional device outputs (see above)
 *   workspace   at least h2o_workspace_bytes(cache, 0) bytes (see the
 *               workspace contract above); may be NULL when that is 0
 * Per unit, with n = min(k, t) valid slots (H2O blog §2.2, §2.3; analysis
 * page §3.2):
 *   1. s_j = q . key_j / sqrt(head_dim) over the n valid slots and the new
 *      token; p = softmax(s); out = sum_j p_j value_j.
 *   2. acc_score[j] += p_j for every valid slot (one fp32 add each); the new
 *      token's score is its own p.
 *   3. If n < k the new token takes slot n. Otherwise the victim is the slot
 *      with the smallest (acc_score, slot_pos), compared lexicographically,
 *      among slots with slot_pos <= t - k_local, and the new token's K/V,
 *      position and score overwrite that slot in place.
 */
h2o_status h2o_decode_step(const h2o_cache_desc* cache, int64_t t, const void* q,
                           const void* k_new, const void* v_new, float* out,
                           const h2o_decode_aux* aux, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * h2o_prefill_ragged - h2o_prefill for a batch whose sequences have their own
 * prompt lengths (the pages' summarisation runs use prompts of varying length;
 * H2O blog §3.2.2).
 *   T_max       rows stored per sequence: q, k, v, out and colsum_out are laid
 *               out as in h2o_prefill with T = T_max
 *   lens        [batch] int32 device array, 4-byte aligned: sequence b's prompt
 *               is its first lens[b] rows (0 <= lens[b] <= T_max; values outside
 *               are clamped to that range on the device, never checked on the host)
 *   workspace   at least h2o_workspace_bytes(cache, T_max) bytes
 * Every unit of sequence b is prefilled and seeded exactly as h2o_prefill does
 * with T = lens[b]; rows lens[b] .. T_max - 1 of out and colsum_out are not
 * written. A sequence with lens[b] = 0 gets every slot marked free. The other
 * arguments, errors and limits are those of h2o_prefill (with T = T_max).
 */
h2o_status h2o_prefill_ragged(const h2o_cache_desc* cache, const void* q, const void* k,
                              const void* v, int32_t T_max, const int32_t* lens, float* out,
                              float* colsum_out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * h2o_decode_step_ragged - h2o_decode_step for a batch whose sequences sit at
 * their own positions.
 *   t           [batch] int32 device array, 4-byte aligned: sequence b's token
 *               goes to position t[b] (clamped to [0, H2O_MAX_POSITION - 1] on
 *               the device); successive calls must advance every t[b] by one,
 *               which the caller does (the library keeps no state)
 * Every unit of sequence b takes exactly the step h2o_decode_step takes at
 * t = t[b]. The other arguments and errors are those of h2o_decode_step.
 */
h2o_status h2o_decode_step_ragged(const h2o_cache_desc* cache, const int32_t* t, const void* q,
                                  const void* k_new, const void* v_new, float* out,
                                  const h2o_decode_aux* aux, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * h2o_decode_step_noalloc - h2o_decode_step for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, serving
 * loops that must not allocate, harnesses that forbid it. Same arguments,
 * results and checks as h2o_decode_step without workspace / workspace_bytes;
 * the same kernels run. It allocates nothing: the scratch that a decode
 * spreading a unit's slots over several workgroups needs lives in a static
 * device array of H2O_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends. A shape that needs more
 * (h2o_workspace_bytes(cache, 0) > H2O_NOALLOC_SCRATCH_BYTES) returns
 * H2O_ERR_UNSUPPORTED and enqueues nothing. The stream must belong to the
 * current device (else H2O_ERR_INVALID). Every call on one GPU shares that
 * GPU's array (its contents on entry never matter), so calls that can overlap
 * on one GPU — on different streams, or from different threads — race and
 * give undefined results; order them on one stream. The first call on a GPU
 * looks up the array's device address (hipGetSymbolAddress); a caller that
 * records the calls in a HIP graph makes one call outside the capture first.
 */
#define H2O_NOALLOC_SCRATCH_BYTES (8u << 20)
h2o_status h2o_decode_step_noalloc(const h2o_cache_desc* cache, int64_t t, const void* q,
                                   const void* k_new, const void* v_new, float* out,
                                   const h2o_decode_aux* aux, void* stream);

/* Static string naming a status code. */
const char* h2o_status_str(h2o_status status);

/* Description of the last failed check or HIP error on the calling thread
 * ("" if none). The pointer stays valid until the next call on that thread. */
const char* h2o_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* H2O_H_ */
