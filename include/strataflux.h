/*
 * strataflux.h -- C ABI of libstrataflux.so: the refined low-bit decode step on
 * AMD MI355X (gfx950).
 *
 * What is computed (the method, per the pages gathered about StrataFlux):
 *   - rag-lover.com StrataFlux summary, explainer dialogue (解説): weights and the
 *     KV cache stay on the GPU in low-bit form; extra precision is fetched from
 *     host memory as a few additional bits that subdivide the interval between
 *     resident low-bit levels ("nested refinement"), not as a full FP16 copy;
 *     weight refinements are chosen by input-activation magnitude, KV refinements
 *     by the attention weight computed from the low-bit keys; fetched precision
 *     is cached on the GPU and reused across decode steps.
 *   - the same page, limitations section (限界と未検証の範囲): on a cache miss the
 *     value stays at its resident low-bit precision.
 *   - "StrataFlux: Memory-Hierarchy-Native Low-Bit LLM Inference" (arXiv
 *     2611.08363), abstract: only selected precision is streamed, delivery
 *     overlaps computation, and fetched precision is reused across steps.
 *
 * Number format (the pages leave it open; this library fixes it):
 *   per group of 128 consecutive values, an asymmetric uniform code of B = b + r
 *   bits: z = fp16(min), s = fp16((max - min) / (2^B - 1)) (one round-to-nearest-
 *   even of the fp64 quotient), c = clamp(rint((x - z) / s), 0, 2^B - 1) in fp64,
 *   c = 0 for a group whose s is 0.  The resident code is c >> r, dequantised as
 *   z + (s * 2^r) * (c >> r); the refinement code is c & (2^r - 1), and with it the
 *   value is z + s * c.  Codes are packed as LSB-first little-endian bit streams.
 *   The per-group parameters are stored as one 32-bit word per group:
 *   bits 0..15 = s (fp16), bits 16..31 = z (fp16).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller (allocated by the
 *     caller, e.g. with PyTorch), unless the argument says "host".  The library
 *     never frees caller memory.  Library objects (sf_refine_cache, sf_workspace)
 *     are opaque handles with create/destroy.
 *   - Calls are stream-ordered: they enqueue work on the given HIP stream
 *     (sf_stream = hipStream_t, NULL = the default stream) and return.
 *   - Calls that take a workspace or a cache allocate no memory; only the
 *     *_create calls allocate.  A workspace must not be used by two calls that
 *     can run at the same time (one stream at a time).
 *   - Errors: argument and shape checks are synchronous and return SF_EINVAL /
 *     SF_EUNSUPPORTED / SF_ENOMEM; a failed HIP call returns SF_EHIP.  Details
 *     are in sf_last_error() (per thread).  Device-side faults surface at the
 *     caller's next synchronisation.  A refinement miss is not an error.
 */
#ifndef STRATAFLUX_H
#define STRATAFLUX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SF_ABI_VERSION 1

typedef int32_t sf_status;
#define SF_OK 0
#define SF_EINVAL 1
#define SF_EUNSUPPORTED 2
#define SF_ENOMEM 3
#define SF_EHIP 4
#define SF_ESTATE 5

typedef void* sf_stream; /* hipStream_t */

/* b resident bits, r refinement bits, group size (must be 128 on the GPU). */
typedef struct {
  int32_t b, r, group;
} sf_qfmt;

/* Layouts of the refinement codes written by sf_quantize_nested. */
#define SF_REFINE_CHANNEL_MAJOR 0 /* weights: [cols][rows*r/8]; unit k = refinement
                                     bits of input channel k over all rows */
#define SF_REFINE_ROW_MAJOR 1     /* [rows][cols*r/8]; unit = one row */

/* A nested-quantised weight matrix, torch layout [n_out][k_in], groups along k_in. */
typedef struct {
  const uint8_t* resident; /* [n_out][k_in*b/8] packed resident codes */
  const uint32_t* sz;      /* [n_out][k_in/128] (scale fp16 | zero fp16 << 16) */
  int64_t n_out, k_in;
  sf_qfmt fmt;
} sf_qweight;

/* A nested-quantised KV cache, one group per token-head (head_dim = 128).
 * k_res, v_res: [batch][n_kv_heads][t_cap][head_dim*b/8]; k_sz, v_sz:
 * [batch][n_kv_heads][t_cap] words as above.  Tokens [0, t_len) are valid.
 * KV refinement unit of (batch i, kv head h, token t): unit id
 * (i*n_kv_heads + h)*t_cap + t, bytes = K refinement stream (head_dim*r/8) followed
 * by the V refinement stream (head_dim*r/8). */
typedef struct {
  uint8_t* k_res;
  uint32_t* k_sz;
  uint8_t* v_res;
  uint32_t* v_sz;
  int32_t batch, n_kv_heads, head_dim, t_len, t_cap;
  sf_qfmt fmt;
} sf_qkv;

typedef struct sf_refine_cache sf_refine_cache;
typedef struct sf_workspace sf_workspace;

/* ---- misc ------------------------------------------------------------------ */
int32_t sf_abi_version(void);
const char* sf_status_string(sf_status s);
const char* sf_last_error(void);

/* Device workspace for the refined GEMV and attention calls.  `bytes` from
 * sf_workspace_bytes_gemv / sf_workspace_bytes_attn (take the maximum over the
 * calls that share it).  Its control block is zeroed at creation; every call
 * leaves it as it found it. */
sf_status sf_workspace_create(size_t bytes, sf_workspace** out);
sf_status sf_workspace_destroy(sf_workspace* ws);
size_t sf_workspace_bytes_attn(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t t_len, int32_t k_sel);
/* Returns SF_ESTATE if a device-side wait timed out in a call that used this
 * workspace since the last check; the affected rows then carry no refinement.
 * After a timeout it also clears every flag and counter in the workspace, so the
 * next call starts from a clean state.  Synchronises the device. */
sf_status sf_workspace_check(sf_workspace* ws);
/* Test hook: the number of polls a bounded device wait of calls on this workspace
 * makes before it gives up (0 = the default, about a second).  A small value makes
 * the waits give up early, from the host, without any kernel hanging; the calls then
 * fall back to resident precision where they gave up and sf_workspace_check reports
 * it.  Synchronises the device. */
sf_status sf_workspace_set_spin_limit(sf_workspace* ws, uint32_t polls);

/* ---- a1: nested quantisation ----------------------------------------------- */
/* Quantise x fp32 [rows][cols] (cols % 128 == 0) to the nested format above.
 * Writes resident [rows][cols*b/8], sz [rows][cols/128] and the refinement codes in
 * `refine_layout`; for SF_REFINE_CHANNEL_MAJOR rows*r must be a multiple of 32.
 * `refine` may be NULL (r == 0, or refinement not wanted).  Format: see top. */
sf_status sf_quantize_nested(const float* x, int64_t rows, int64_t cols, sf_qfmt fmt,
                             int32_t refine_layout, uint8_t* resident, uint32_t* sz,
                             uint8_t* refine, sf_stream stream);

/* Test helper: dequantise to fp32 [rows][cols].  which = 0: resident value
 * z + (s*2^r)*(c>>r); which = 1: full value z + s*c (needs `refine` in
 * `refine_layout`).  Each value is one round-to-nearest-even of the exact value. */
sf_status sf_debug_dequantize(const uint8_t* resident, const uint32_t* sz,
                              const uint8_t* refine, int64_t rows, int64_t cols,
                              sf_qfmt fmt, int32_t refine_layout, int32_t which,
                              float* out, sf_stream stream);

/* ---- a7: KV append --------------------------------------------------------- */
/* Quantise n_tok new tokens of K and V (fp32 [batch][n_kv_heads][n_tok][head_dim])
 * into positions [t0, t0 + n_tok) of `kv` (t0 + n_tok <= t_cap; kv->t_len is not
 * changed by the call).  Their refinement units (layout of sf_qkv) are written
 * to refine_out (device, may be NULL): the unit of (batch i, head h, new token j)
 * at refine_out + ((i*n_kv_heads + h)*refine_ld + j) * unit_bytes.  refine_ld =
 * n_tok packs them; refine_ld = t_cap with refine_out pointing at unit t0 of a
 * store laid out like the cache writes them in place.  Per (batch, head, token)
 * the K row and the V row are one group each. */
sf_status sf_kv_append(const float* k_new, const float* v_new, int32_t n_tok, int32_t t0,
                       const sf_qkv* kv, uint8_t* refine_out, int64_t refine_ld,
                       sf_stream stream);

/* ---- a3, a13: refinement slot cache ---------------------------------------- */
/* One pool per refined tensor.  Units are fixed-size byte strings, unit ids
 * 0..n_units-1; host_store (pinned host memory, from hipHostMalloc or torch
 * pin_memory, kept alive by the caller) holds every unit, [n_units][unit_bytes].
 * Fills read it directly from the device over PCIe; create fails with SF_EINVAL
 * if a pool with slots has a store that is not pinned.
 * If device_store is non-NULL, the pool is a resident pool: capacity must equal
 * n_units, device_store [n_units][unit_bytes] (caller device memory) already
 * holds every unit, unit u lives in slot u, and the pool never misses.
 * SSD tier (rag-lover.com StrataFlux summary, TL;DR and limitations section: the
 * extra precision may also sit on an SSD, whose 2 KB random reads are slow; paper
 * abstract, arXiv 2611.08363: host RAM and solid-state drives): if store_file is
 * non-NULL (and host_store NULL), the units are read from that file instead, unit
 * u at byte store_offset + u * unit_bytes.  A fill reads each unit it installs
 * with its own positioned read (direct I/O, bypassing the page cache, where the
 * file system allows it; up to 8 reads in flight) into pinned staging the cache
 * owns, then copies staging to slots as for a host store.  The file must hold
 * every unit when the cache is created and must not change while it exists. */
typedef struct {
  int64_t unit_bytes; /* multiple of 4 */
  int64_t n_units;
  int64_t capacity; /* device slots, 0 <= capacity <= n_units */
  const uint8_t* host_store;
  uint8_t* device_store;
  int32_t max_lookup; /* most unit ids one step looks up in this pool */
  const char* store_file; /* NULL: the store is host_store (or device_store) */
  int64_t store_offset;
  int32_t lead_slots; /* device slots beyond capacity that sf_refine_cache_prefetch fills */
} sf_pool_desc;

#define SF_CACHE_DETERMINISTIC 0 /* fill completes before the next step's lookups */
#define SF_CACHE_ASYNC 1         /* fills land when their copy has finished */

/* Creates the cache on the current device.  Lookups at step t mark hits as used
 * at t and queue misses; sf_refine_cache_fill (end of step t) installs the queued
 * misses in the order they were looked up: into a free slot, else in place of the
 * resident unit with the smallest (last use, unit id) among those last used
 * before t, else the miss is dropped; at most max_fill units per pool per fill
 * (0 = no cap).  Installed units count as used at t. */
sf_status sf_refine_cache_create(const sf_pool_desc* pools, int32_t n_pools, int32_t mode,
                                 int32_t max_fill, sf_refine_cache** out);
sf_status sf_refine_cache_destroy(sf_refine_cache* c);

/* Looks up n device unit ids of `pool`; writes the slot of each (or -1) to
 * slot_out (device, may be NULL) and records the lookup for the next fill. */
sf_status sf_refine_cache_lookup(sf_refine_cache* c, int32_t pool, const int32_t* unit_ids,
                                 int32_t n, int32_t* slot_out, sf_stream compute);

/* End of a decode step: reads the step's lookups of every pool (one kernel into a
 * pinned mirror, then one wait on `compute`), runs the replacement policy, and
 * installs the missed units of every pool: the victims are unmapped on `compute`,
 * one kernel on `side` copies the new units from the pinned host stores into
 * their slots, and they are mapped on `compute` behind that copy.
 * Deterministic mode: returns after the new units are visible to work enqueued
 * later on `compute`.  Async mode (the host never waits for the step in flight):
 * the call at the end of step t copies step t's lookups to the host and runs the
 * policy on step t-1's (replacement decisions as of step t-1); their copy runs on
 * `side` behind step t's work and the next call maps them, so they serve lookups
 * from step t+2 on.  n_filled (host, may be NULL):
 * units installed or queued for install by this call.  SF_ESTATE if a pool's
 * lookups of the step exceeded its max_lookup (the excess was not recorded). */
sf_status sf_refine_cache_fill(sf_refine_cache* c, sf_stream compute, sf_stream side,
                               int64_t* n_filled);

/* Host-side statistics since creation: lookups, hits, units installed, bytes
 * copied host-to-device; per pool if pool >= 0, all pools if pool < 0. */
sf_status sf_refine_cache_stats(sf_refine_cache* c, int32_t pool, int64_t* lookups,
                                int64_t* hits, int64_t* installed, int64_t* h2d_bytes);

/* Fetch lead (rag-lover.com StrataFlux summary, explainer dialogue (解説), fetch lead /
 * fetch lag passage: the channels a block will need are predicted from the
 * previous block's residual stream and fetched ahead of it).  The pool's
 * lead_slots ring slots come to hold the units named by unit_ids (device [n],
 * distinct): ring units named again stay; every other ring slot is emptied (its
 * unit unmapped unless an LRU slot serves it); the named units found in no slot,
 * in the order given, are copied from the pinned host store into the empty ring
 * slots (ascending) and mapped, as many as there are empty slots.  Three kernels
 * on `stream` (a side stream: work on the compute stream that looks these units
 * up must wait for it; nothing else may look up or fill this pool meanwhile).
 * Lookups that find a unit in a ring slot are hits that do not count as LRU use;
 * fills never evict ring slots.  SF_EINVAL if the pool has no lead slots. */
sf_status sf_refine_cache_prefetch(sf_refine_cache* c, int32_t pool, const int32_t* unit_ids, int32_t n,
                                   sf_stream stream);

/* Fetch lag (rag-lover.com StrataFlux summary, explainer dialogue (解説), fetch lead /
 * fetch lag passage: a refinement's addition to the output may wait for a later
 * update, so that its transfer overlaps computation).  For a refined GEMV that
 * ran with selection sel [k_sel] and per-channel slots hit [k_sel] (its sel_out
 * and hit_out; -1 = missed), writes the contribution the missed channels would
 * have made, delta_out[b][n] = sum over j with hit[j] < 0 of
 * x[b][sel[j]] * s[n][sel[j]/128] * c_lo[n][sel[j]], fp32 [batch][n_out]
 * (overwritten; zero if nothing missed).  The refinement bits are read straight
 * from the pool's pinned host store over PCIe (a resident pool reads its device
 * store); the pool's units must be w's channel-major refinement units.  Run it on
 * a side stream and add delta_out into the output's next update (sf_residual_add)
 * once it is done.  batch 1..16; a pool whose store is a file: SF_EUNSUPPORTED. */
sf_status sf_refine_lag_delta(sf_refine_cache* c, int32_t pool, const sf_qweight* w, const uint16_t* x_f16,
                              int32_t batch, int32_t k_sel, const int32_t* sel, const int32_t* hit,
                              float* delta_out, sf_stream stream);

/* FP16 fetch, a comparison variant (rag-lover.com StrataFlux summary, "既存手法との
 * 違い": fetching FP16 values instead of refinement bits).  The pool's units are
 * w's columns as fp16 (unit k = fp16(W[0..n_out)[k]), 2 * n_out bytes).  After a
 * resident GEMV that selected sel [k_sel] (sf_refined_gemv with cache NULL and
 * sel_out) and a lookup of sel in this pool (sf_refine_cache_lookup -> slot), adds
 * y[b][n] += sum over j with slot[j] >= 0 of x[b][sel[j]] * (w16[n][sel[j]] -
 * resident[n][sel[j]]), so that the fetched columns hold their fp16 value.
 * batch 1..16. */
sf_status sf_fp16_fetch_delta(sf_refine_cache* c, int32_t pool, const sf_qweight* w, const uint16_t* x_f16,
                              int32_t batch, int32_t k_sel, const int32_t* sel, const int32_t* slot, float* y,
                              sf_stream stream);

/* Reads of a pool with a store file (pool < 0: all such pools) since creation:
 * units read, bytes read, the median and 99th percentile of one unit's read time
 * (microseconds, over the last 65536 reads), and the wall time fills spent
 * reading (milliseconds).  All zero if no pool reads from a file. */
sf_status sf_refine_cache_io_stats(sf_refine_cache* c, int32_t pool, int64_t* reads, int64_t* bytes,
                                   double* p50_us, double* p99_us, double* read_ms);

/* Test helper: writes the resident unit ids of `pool` (ascending) to ids (host,
 * room for capacity entries) and their count to *n. */
sf_status sf_refine_cache_resident(sf_refine_cache* c, int32_t pool, int64_t* ids, int64_t* n);

/* ---- a2-a6: refined GEMV ----------------------------------------------------- */
/* One matrix of a fused GEMV call.  All ops of a call share x, k_in and fmt. */
typedef struct {
  sf_qweight w;
  int32_t pool;     /* cache pool of this matrix (unit k = input channel k), -1 = none */
  float* y;         /* [batch][n_out] fp32 */
  int32_t* hit_out; /* optional [k_sel]: slot of each selected channel, -1 = miss */
} sf_gemv_op;

/* Workspace bytes for sf_refined_gemv(ops, n_ops, ..., batch, k_sel, ...): the
 * selection, the slot lists and, for the batched kernel, the partial outputs of
 * its channel slices ([slices][min(batch, 16)][padded rows] fp32).  The batched
 * kernel's plan depends on the CU count of the current device. */
size_t sf_workspace_bytes_gemv(const sf_gemv_op* ops, int32_t n_ops, int32_t batch, int32_t k_sel);

/* y = x W_eff^T for each op, x fp16 [batch][k_in] (batch >= 1), where W_eff uses
 * the full (b+r)-bit value on the selected channels whose refinement unit is in
 * the cache (a hit) and the resident value everywhere else.
 * Selection: if sel_in (device [k_sel], ascending, distinct) is NULL, the k_sel
 * channels of largest max-over-batch |x|, ties to the lower index.  sel_out
 * (device [k_sel], may be NULL) receives the selection, ascending.  k_sel = 0 is
 * the unrefined low-bit GEMV.  cache may be NULL (every selection misses).
 * A computed selection (sel_in NULL, 0 < k_sel < k_in) needs k_in <= 32768
 * (SF_EUNSUPPORTED otherwise).  Launches at batch 1-2: one; its first workgroup
 * computes the selection while the others stream the resident codes, or, with
 * sel_in given, every workgroup looks up its hits itself.  At batch >= 3: the
 * selection with its lookups, then for b in {1, 2, 4, 8} the batched MFMA kernel,
 * one launch per 16 batch rows, otherwise one launch per 2 batch rows.
 * Test hooks (environment): SF_GEMV_SPLIT=0 / 2 forces the variant where every
 * workgroup selects / the variant with x staged in LDS; SF_GEMV_ROWS_PER_WAVE=4 / 8;
 * SF_GEMV_MFMA=0 / 1, SF_GEMV_MFMA_RT, SF_GEMV_MFMA_SLICES force the batched
 * kernel's use and plan. */
sf_status sf_refined_gemv(const sf_gemv_op* ops, int32_t n_ops, const uint16_t* x_f16,
                          int32_t batch, int32_t k_sel, const int32_t* sel_in,
                          int32_t* sel_out, sf_refine_cache* cache, sf_workspace* ws,
                          sf_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): sf_refined_gemv without a
 * workspace.  Same arguments, semantics and kernels; the selection, slot lists,
 * hand-off words and batched partials live in a library-owned scratch array of
 * 8 MiB per device (a static device variable, held by each device the library runs
 * on until the process ends).  Allocates nothing and calls no allocating routine.
 * Returns SF_ENOMEM, before any launch, if the call would need more scratch than
 * that (sf_workspace_bytes_gemv for the same arguments above 8 MiB).  Every call on
 * a device shares that device's array and first clears its flags and counters
 * (one small kernel on `stream`): calls that can run at the same time on one device
 * (other streams, other host threads) race and must not be issued. */
sf_status sf_refined_gemv_noalloc(const sf_gemv_op* ops, int32_t n_ops, const uint16_t* x_f16,
                                  int32_t batch, int32_t k_sel, const int32_t* sel_in,
                                  int32_t* sel_out, sf_refine_cache* cache, sf_stream stream);

/* ---- a8-a12: refined GQA decode attention ------------------------------------ */
/* out fp32 [batch][n_q_heads][head_dim] for q fp16 [batch][n_q_heads][head_dim]
 * over tokens [0, kv->t_len).  Query head h reads KV head h / (n_q/n_kv).
 * Per (batch, kv head): logits from the resident keys, softmax per query head,
 * token score = that softmax summed over the kv head's query heads; the k_sel
 * tokens of largest score (ties to the lower token) are selected (or sel_in,
 * device [batch][n_kv][k_sel], ascending and distinct per KV head), looked up
 * in `pool`, and for the hits
 * both the key and the value use the full (b+r)-bit value; the output softmax is
 * over all tokens after that replacement.  sel_out / hit_out (device
 * [batch][n_kv][k_sel], may be NULL) receive the selection and slots.
 * t_len <= 1048576.  Workspaces may be shared by calls on one stream, not by
 * calls that can run at the same time. */
sf_status sf_refined_attn_decode(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                 float softmax_scale, int32_t k_sel, const int32_t* sel_in,
                                 sf_refine_cache* cache, int32_t pool, float* out,
                                 int32_t* sel_out, int32_t* hit_out, sf_workspace* ws,
                                 sf_stream stream);

/* The decode step's KV append and attention in one call (rag-lover.com StrataFlux
 * summary, explainer dialogue (解説): the new token's K and V join the low-bit cache
 * and the step attends over it).  Same result as sf_kv_append(k_new, v_new, 1,
 * kv->t_len - 1, kv, refine_out, refine_ld, stream) followed by
 * sf_refined_attn_decode(q_f16, n_q_heads, kv, ...) on the same stream: kv->t_len
 * counts the new token, which is quantised into position t_len - 1 (codes, sz words
 * and, when refine_out is non-NULL, its refinement units at refine_out + (i *
 * n_kv_heads + h) * refine_ld * unit_bytes for batch i, head h) by the attention's
 * own first pass, saving a launch.  k_new, v_new: device fp32 [batch][n_kv_heads]
 * [head_dim].  out_f16 (device, may be NULL): out again as fp16 bits (round to
 * nearest even, as sf_to_f16), the input of the o projection, written by the same
 * kernel that writes out.  The nested variant only; errors as
 * sf_refined_attn_decode, and SF_EINVAL for null k_new / v_new or refine_ld < 1
 * with refine_out. */
sf_status sf_refined_attn_decode_append(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                        const float* k_new, const float* v_new, uint8_t* refine_out,
                                        int64_t refine_ld, float softmax_scale, int32_t k_sel,
                                        const int32_t* sel_in, sf_refine_cache* cache, int32_t pool,
                                        float* out, uint16_t* out_f16, int32_t* sel_out,
                                        int32_t* hit_out, sf_workspace* ws, sf_stream stream);

/* Comparison variants of the refined attention (rag-lover.com StrataFlux summary,
 * "既存手法との違い": the paper compares nested refinement with SpeCache, which
 * replaces selected tokens by their FP16 values, and with sparse attention, which
 * drops the unselected tokens).  Same arguments, selection and cache semantics as
 * sf_refined_attn_decode; `variant`:
 *   SF_ATTN_NESTED           sf_refined_attn_decode itself;
 *   SF_ATTN_FP16_TOKENS      a selected token that hits uses fp16 K and V from its
 *                            unit (512 bytes: K[0..128) fp16, then V[0..128) fp16)
 *                            in place of its resident vectors, for its logit and its
 *                            value; the softmax runs over all tokens (fmt.r may be 0);
 *   SF_ATTN_DROP_UNSELECTED  only the selected tokens are attended (softmax over
 *                            them), each at (b+r) bits if it hits, else resident;
 *                            needs k_sel >= 1.
 * The pool's units must be of the variant's kind (SF_EINVAL otherwise). */
#define SF_ATTN_NESTED 0
#define SF_ATTN_FP16_TOKENS 1
#define SF_ATTN_DROP_UNSELECTED 2
sf_status sf_attn_decode_variant(const uint16_t* q_f16, int32_t n_q_heads, const sf_qkv* kv,
                                 float softmax_scale, int32_t k_sel, const int32_t* sel_in,
                                 sf_refine_cache* cache, int32_t pool, float* out,
                                 int32_t* sel_out, int32_t* hit_out, sf_workspace* ws, sf_stream stream,
                                 int32_t variant);

/* ---- a14: decode-step glue ------------------------------------------------- */
/* A decoder step around the refined GEMV and attention, after the public
 * Llama-3.1 / Qwen3 layer definitions (the pages describe only the refined ops):
 * fp32 residual stream, fp16 GEMV inputs, RMSNorm, per-head q/k RMSNorm (Qwen3),
 * rotate-half rotary embedding, SwiGLU, greedy argmax.  All pointers are device
 * memory owned by the caller; every call is one stream-ordered launch. */

/* h_out[b][:] = table_f16[ids[b]][:] as fp32 ([batch][hidden]).  table [vocab][hidden].
 * An id outside [0, vocab) gives a row of zeros. */
sf_status sf_embed(const uint16_t* table_f16, int64_t vocab, int32_t hidden, const int32_t* ids,
                   int32_t batch, float* h_out, sf_stream stream);

/* Residual add and RMSNorm, per batch row of `hidden` values: if y is non-NULL,
 * h += y (h updated in place); then x_f16 = fp16(h / sqrt(mean(h^2) + eps) * w),
 * rounded to nearest even.  h, y [batch][hidden] fp32; w [hidden] fp32. */
sf_status sf_add_rmsnorm(float* h, const float* y, const float* w, int32_t batch, int32_t hidden,
                         float eps, uint16_t* x_f16, sf_stream stream);

/* Query / key heads (head_dim 128) at position `pos`: q [batch][n_q][128] and
 * k [batch][n_kv][128] fp32 (the GEMV outputs).  If q_norm_w / k_norm_w ([128] each,
 * both or neither) are given, each head is first RMS-normalised (eps) and scaled.
 * Then the rotary embedding: dims i and i+64 rotate by pos * theta^(-2i/128)
 * (angles in fp64).  Writes the queries as fp16 to q_f16 [batch][n_q][128] and the
 * keys as fp32 to k_out [batch][n_kv][128] (the input of sf_kv_append; may be k). */
sf_status sf_qk_rope(const float* q, const float* k, int32_t batch, int32_t n_q, int32_t n_kv,
                     const float* q_norm_w, const float* k_norm_w, float eps, int32_t pos,
                     float theta, uint16_t* q_f16, float* k_out, sf_stream stream);

/* Producers of a refined GEMV's input that also select its channels (rag-lover.com
 * StrataFlux summary, explainer dialogue: weight refinements are chosen by
 * input-activation magnitude).  Each is one launch of one workgroup that writes the
 * fp16 input x [batch][n] exactly as the call named in its comment does and, in the
 * same launch, the k_sel channels of largest max-over-rows |x| (ties to the lower
 * channel) in ascending order to sel_out (device [k_sel]; k_sel = 0 selects nothing,
 * k_sel = n every channel).  Passing sel_out as the GEMV's sel_in lets the GEMV start
 * with its selection ready.  1 <= batch <= 16, n % 8 == 0, n <= 32768, every tensor
 * 16-byte aligned (SF_EINVAL otherwise).
 * sf_add_rmsnorm_select: sf_add_rmsnorm (hidden = n).
 * sf_swiglu_select: sf_swiglu over gate, up [batch][n].
 * sf_to_f16_select: sf_to_f16 of x [batch][n]. */
sf_status sf_add_rmsnorm_select(float* h, const float* y, const float* w, int32_t batch, int32_t hidden, float eps,
                                uint16_t* x_f16, int32_t k_sel, int32_t* sel_out, sf_stream stream);
sf_status sf_swiglu_select(const float* gate, const float* up, int32_t batch, int32_t n, uint16_t* act_f16,
                           int32_t k_sel, int32_t* sel_out, sf_stream stream);
sf_status sf_to_f16_select(const float* x, int32_t batch, int32_t n, uint16_t* out_f16, int32_t k_sel,
                           int32_t* sel_out, sf_stream stream);

/* act_f16[i] = fp16(silu(gate[i]) * up[i]), silu(x) = x / (1 + e^-x); n elements. */
sf_status sf_swiglu(const float* gate, const float* up, int64_t n, uint16_t* act_f16, sf_stream stream);

/* out_f16[i] = fp16(x[i]) (nearest even), n elements. */
sf_status sf_to_f16(const float* x, int64_t n, uint16_t* out_f16, sf_stream stream);

/* h[i] += d[i], n elements (a residual update with a late contribution, see
 * sf_refine_lag_delta). */
sf_status sf_residual_add(float* h, const float* d, int64_t n, sf_stream stream);

/* ids[b] = index of the largest logits[b][:] ([batch][vocab] fp32), the lowest index
 * among equal maxima; NaN values are never chosen. */
sf_status sf_argmax(const float* logits, int32_t batch, int64_t vocab, int32_t* ids, sf_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* STRATAFLUX_H */
