/*
 * sdpa.h - C ABI of the MI355X (gfx950) fused scaled-dot-product attention
 * forward library, libsdpa.so.
 *
 *   out = softmax(scale * Q K^T + mask) V
 *
 * The operation is the one tested by nuvec-core "tests/fast.rs"
 * (attention_fallback_matches_a_direct_formula: scores scale * q.k, the row
 * maximum subtracted before exp, weights divided by their sum, applied to v),
 * with the masking and all-masked-row semantics of lattice-inference
 * "src/attention/flash.rs" (run_tiled_attention_head: masked keys get zero
 * weight; a row that sees no key outputs zeros) and its grouped-query head
 * mapping (kv_head_index: query head h reads key/value head h / (Hq/Hkv)).
 *
 * Every tensor pointer is a DEVICE pointer to a contiguous row-major array
 * and must be 16-byte aligned (the mask and sinks excepted). The caller owns
 * every buffer. `out` must not overlap any input.
 *
 * Errors are return codes; nothing aborts, throws or prints. After an error,
 * sdpa_last_error() returns a message naming the offending argument.
 */
#ifndef SDPA_H
#define SDPA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v, out and sinks (all the same type). */
enum { SDPA_F32 = 0, SDPA_F16 = 1, SDPA_BF16 = 2 };

/* Mask kinds.
 * SDPA_MASK_NONE   every key is visible.
 * SDPA_MASK_CAUSAL bottom-right aligned: query i sees key j iff j <= i + Lk - Lq
 *                  (nuvec-core tests/fast.rs, direct-formula test). With Lq > Lk
 *                  the first Lq - Lk rows see nothing and output zeros.
 * SDPA_MASK_BOOL   a device uint8 matrix [Lq, Lk], nonzero = visible, shared by
 *                  every batch item and head (nuvec-core tests/attention_plan.rs,
 *                  attention(); tests/fast.rs, window_mask).
 * SDPA_MASK_ADDITIVE  values in the element type added to the scaled scores,
 *                  scale * q.k + mask[b, h, i, j], through a strided view that may
 *                  broadcast over batch items and heads (tests/fast.rs,
 *                  attention_kernels_match_the_fallback: an additive [1, Hq, Lq, Lk]
 *                  mask). A -inf entry drops its key; a row of -inf outputs zeros.
 *                  Only sdpa_forward_strided takes one (sdpa_plan plans it). */
enum { SDPA_MASK_NONE = 0, SDPA_MASK_CAUSAL = 1, SDPA_MASK_BOOL = 2, SDPA_MASK_ADDITIVE = 3 };

/* Return codes. */
enum {
  SDPA_OK = 0,
  SDPA_ERR_INVALID = -1,     /* an argument is malformed (shape, pointer, dtype, overflow) */
  SDPA_ERR_UNSUPPORTED = -2, /* well-formed but not built: a head-size pair outside the list below */
  SDPA_ERR_HIP = -3          /* the HIP runtime reported an error while enqueuing */
};

/* Routes a call can take (sdpa_plan_t.route). */
enum {
  SDPA_ROUTE_EMPTY = 0,     /* B*Hq*Lq*Dv == 0: nothing to do, no launch */
  SDPA_ROUTE_ZERO_FILL = 1, /* Lk == 0: out is filled with zeros by one small kernel */
  SDPA_ROUTE_PREFILL = 2,   /* tiled online-softmax kernel over query blocks */
  SDPA_ROUTE_DECODE = 3     /* split-key first pass over key blocks, then a log-sum-exp reduce */
};

/* The plan of one call: a pure function of the shapes, mask kind, sinks flag and dtype. */
typedef struct sdpa_plan_t {
  int32_t route;          /* SDPA_ROUTE_* */
  int32_t kernels;        /* kernel launches the call enqueues */
  int32_t rows_per_wave;  /* query rows one wavefront carries (MFMA tile height). Prefill: 16 on
                             the key-split kernel (f16/bf16, (D, Dv) in {(192,192), (192,128),
                             (256,256)} with every mask kind, (128,128) with an additive mask,
                             and (D, Dv) in {(64,64), (80,80), (96,96), (128,128), (96,64)} when the
                             pipelined kernel's grid for one batch item would have fewer than 256
                             workgroups); 32 on the pipelined kernel (other f16/bf16
                             calls with (D, Dv) in {(64,64), (80,80), (96,96), (128,128), (96,64)},
                             no additive mask);
                             else the generic kernel's 32 (heads up to 128 wide) or 16 (wider
                             heads; and f32 calls whose 32-row grid for one batch item would have
                             fewer than 256 workgroups) */
  int32_t waves;          /* wavefronts per workgroup of the first kernel */
  int32_t block_n;        /* keys per tile */
  int32_t heads_per_group;/* prefill: query heads sharing one workgroup's K/V tiles;
                             decode: query heads packed into one wavefront (Hq/Hkv) */
  int64_t keys_per_split; /* decode: keys per first-pass workgroup (a power of two, 64..1024,
                             from Lk alone so that batch items never change it) */
  int64_t splits;         /* decode: key blocks per (batch, kv head). Prefill: 0, or, for f32 calls
                             whose 32-row grid for one batch item would have fewer than 256
                             workgroups (no additive mask), the waves of a workgroup
                             that split the keys of its one 16-row query block and merge their
                             partial results (heads_per_group is then 1); or 2 on the key-split
                             kernel: two lanes of `waves`/2 wavefronts each take 32 of every
                             `2 * block_n` keys and merge at the end */
  int64_t grid[3];        /* workgroups of the attention kernel (decode: its first pass) (x, y, z) */
  int64_t scratch_bytes;  /* device scratch the call uses. Decode: per (batch, kv head, split, packed
                             row) a 16-byte {max, sum} slot and Dv f32 partial outputs. Prefill: 0,
                             except f16/bf16 with a boolean mask outside the key-split kernel,
                             whose mask a first small kernel packs into Lq x ceil(Lk/32) 32-bit
                             words (bit j of word w: key 32w+j); the key-split kernel reads the
                             mask bytes itself */
} sdpa_plan_t;

/*
 * sdpa_forward - enqueue one attention forward on `stream`.
 *
 *   q     [B, Hq,  Lq, D ]   device, dtype
 *   k     [B, Hkv, Lk, D ]   device, dtype
 *   v     [B, Hkv, Lk, Dv]   device, dtype
 *   out   [B, Hq,  Lq, Dv]   device, dtype, written in full
 *   Hq must be a multiple of Hkv; query head h reads kv head h / (Hq / Hkv).
 *   scale  any finite float, applied to q.k as given (1/sqrt(D) is usual).
 *   mask_kind  SDPA_MASK_NONE, _CAUSAL or _BOOL; `mask` is required (device
 *          [Lq, Lk] uint8) iff mask_kind == SDPA_MASK_BOOL and ignored
 *          otherwise. A raw pointer carries no shape: the caller guarantees
 *          Lq*Lk readable bytes. SDPA_MASK_ADDITIVE is SDPA_ERR_INVALID here
 *          (an additive mask needs its strides: sdpa_forward_strided).
 *   sinks  NULL, or device [Hq] in dtype: one logit per query head that joins
 *          the softmax denominator only (no value row) and is not multiplied
 *          by `scale`.
 *   Head sizes (D, Dv): (64,64) (80,80) (96,96) (128,128) (192,192) (256,256)
 *          (512,512) (96,64) (192,128); others -> SDPA_ERR_UNSUPPORTED.
 *   stream a hipStream_t (NULL = the default stream).
 *
 * Computation is float32 inside the kernels (f32 MFMA for SDPA_F32, bf16/f16
 * MFMA with f32 accumulation otherwise); the output is rounded once to dtype.
 * Empty cases: B*Hq*Lq == 0 or Dv == 0 enqueue nothing; Lk == 0 writes zeros.
 * The call is asynchronous: validation errors return before anything is
 * enqueued; a launch failure returns SDPA_ERR_HIP. A given plan gives the
 * same bits run to run, and each batch item's bits do not depend on B.
 * Scratch (decode partials, packed mask bits; sdpa_plan's scratch_bytes)
 * comes from a per-(device, stream) buffer that the library allocates with
 * hipMallocAsync on the stream's first call that needs it. A later call that
 * needs more replaces it with a buffer at least twice as large; the replaced
 * buffer is kept, not freed, until sdpa_release_workspace, so graphs captured
 * earlier on the stream keep valid addresses.
 * Graph capture: a call may be captured (hipStreamBeginCapture) once the
 * stream's buffer is large enough; make one call of at least the plan's
 * scratch_bytes on the same stream, outside the capture, first. A captured
 * call that would need a larger buffer (or the stream's first buffer) returns
 * SDPA_ERR_UNSUPPORTED and enqueues nothing. A captured graph keeps using the
 * buffer of the stream it was captured on: replaying it while other calls on
 * that stream's buffer run (on the stream, or other replays of graphs captured
 * there, on any stream) races with them.
 */
int sdpa_forward(const void* q, const void* k, const void* v, void* out,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                 int64_t D, int64_t Dv, float scale,
                 int mask_kind, const uint8_t* mask, const void* sinks,
                 int dtype, void* stream);

/*
 * sdpa_plan - the route, launch geometry and scratch size sdpa_forward would
 * use for these arguments, validated exactly as sdpa_forward validates them
 * (has_mask / has_sinks stand for non-NULL mask / sinks pointers). Pure: no
 * device work and no allocation. `plan` must be non-NULL; it is written only
 * on SDPA_OK. Mirrors nuvec-core tests/attention_plan.rs (plan_attention: a
 * pure host plan naming the kernels that run and the scratch they hold).
 */
int sdpa_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
              int64_t D, int64_t Dv, int mask_kind, int has_mask, int has_sinks,
              int dtype, sdpa_plan_t* plan);

/*
 * sdpa_forward_windowed - causal attention over a sliding window of keys, as
 * sdpa_forward with mask_kind SDPA_MASK_CAUSAL and no boolean mask, except
 * that query row i (position pos = i + Lk - Lq) reads only the keys j with
 * pos - window < j <= pos: the band of nuvec-core tests/fast.rs (window_mask;
 * windows_run_fused_and_equal_the_boolean_mask). A row whose band holds no key
 * is zero. window must be >= 1 (else SDPA_ERR_INVALID); a window of at least
 * Lk keys is plain causal attention, with the same plan and the same bits as
 * sdpa_forward (window_errors_empty_inputs_and_full_windows). Decode key
 * splits cover only the keys the rows read (attention_plan.rs,
 * windowed_decode_plans_from_the_window_keys). Other arguments, layouts,
 * ownership, errors and asynchrony as for sdpa_forward.
 */
int sdpa_forward_windowed(const void* q, const void* k, const void* v, void* out,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                          int64_t D, int64_t Dv, float scale, int64_t window,
                          const void* sinks, int dtype, void* stream);

/* The plan sdpa_forward_windowed would use; pure, like sdpa_plan. */
int sdpa_plan_windowed(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                       int64_t D, int64_t Dv, int64_t window, int has_sinks,
                       int dtype, sdpa_plan_t* plan);

/*
 * sdpa_paged_forward - attention of a few new query rows per sequence over a
 * paged key/value cache (nuvec-core tests/fast.rs: the paged() cache builder,
 * paged_attention_equals_contiguous_attention,
 * paged_windows_and_sinks_equal_contiguous_attention,
 * paged_attention_clamps_hostile_tables_and_lengths).
 *
 *   q       [B, Hq, Lq, D]                 device, dtype
 *   kcache  [blocks, Hkv, bs, D]           device, dtype
 *   vcache  [blocks, Hkv, bs, Dv]          device, dtype
 *   table   [B, max_blocks] int32          device: sequence b's key j is row
 *           j % bs of block table[b][j / bs]
 *   lengths [B] int32                      device: sequence b's key count
 *   out     [B, Hq, Lq, Dv]                device, dtype, written in full
 *
 * Sequence b is attention over its lengths[b] keys gathered back into order,
 * exactly as sdpa_forward (or sdpa_forward_windowed) over those keys: the
 * causal mask and the window are aligned to lengths[b]. Entries and lengths
 * read from device memory are clamped, never trusted: a length to
 * [0, max_blocks * bs], a table entry to [0, blocks - 1]; only the entries
 * that cover a sequence's (windowed) keys are read, and no block outside the
 * cache. A sequence with no key gives zero rows.
 *   mask_kind  SDPA_MASK_NONE or SDPA_MASK_CAUSAL (a boolean mask is
 *          SDPA_ERR_INVALID).
 *   window 0 for none, else >= 1 with SDPA_MASK_CAUSAL (as in
 *          sdpa_forward_windowed); negative, or positive without the causal
 *          mask, is SDPA_ERR_INVALID.
 *   scale, sinks, head sizes as for sdpa_forward.
 *   dtype  SDPA_F16 or SDPA_BF16: the decode kernels (split-key first pass,
 *          log-sum-exp reduce), for Lq <= 8 and (Hq / Hkv) * Lq <= 32 (larger
 *          query counts are SDPA_ERR_UNSUPPORTED); their key splits follow
 *          the cache capacity max_blocks * bs (or, with a window, the
 *          window's keys), not the lengths, which stay on the device.
 *          SDPA_F32: the f32 tiled kernel over the capacity's key range, any
 *          Lq, reading each K/V row through the table.
 * Ownership, alignment, scratch, errors and asynchrony as for sdpa_forward.
 */
int sdpa_paged_forward(const void* q, const void* kcache, const void* vcache, void* out,
                       const int32_t* table, const int32_t* lengths,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                       int64_t D, int64_t Dv, int64_t blocks, int64_t bs, int64_t max_blocks,
                       float scale, int mask_kind, int64_t window, const void* sinks,
                       int dtype, void* stream);

/* The plan sdpa_paged_forward would use; pure, like sdpa_plan. */
int sdpa_plan_paged(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t D, int64_t Dv,
                    int64_t blocks, int64_t bs, int64_t max_blocks, int mask_kind,
                    int64_t window, int has_sinks, int dtype, sdpa_plan_t* plan);

/*
 * sdpa_paged_write - write n new rows into a paged cache in place
 * (nuvec-core tests/fast.rs, paged_write_matches_the_fallback_and_writes_in_place,
 * paged_write_skips_out_of_range_slots).
 *
 *   cache  [blocks, Hkv, bs, E]  device, dtype; rows written in place
 *   rows   [n, Hkv, E]           device, dtype
 *   slots  [n] int32             device: row r goes to block slots[r] / bs,
 *          position slots[r] % bs, for every head
 * A slot outside [0, blocks * bs) is skipped: nothing is written for it.
 * Two rows with the same slot race (either may win). E * sizeof(dtype) must
 * be a multiple of 16 bytes (else SDPA_ERR_UNSUPPORTED); cache and rows must
 * be 16-byte aligned and must not overlap. n == 0 enqueues nothing. One
 * kernel, no scratch; asynchronous on `stream`.
 */
int sdpa_paged_write(void* cache, const void* rows, const int32_t* slots, int64_t n,
                     int64_t blocks, int64_t Hkv, int64_t bs, int64_t E, int dtype,
                     void* stream);

/* A strided view of a [B, H, L, E] operand: element [b, h, l, e] is at
 * data + (b * stride_b + h * stride_h + l * stride_l + e) elements. The last
 * (feature) axis is contiguous. */
typedef struct sdpa_view_t {
  const void* data;
  int64_t stride_b, stride_h, stride_l;
} sdpa_view_t;

/*
 * sdpa_forward_strided - sdpa_forward (and sdpa_forward_windowed) over strided
 * views, and the only call that takes an additive mask: q, k and v may be
 * views such as a transposed [B, L, H, D] array or a slice of a longer cache
 * (nuvec-core tests/fast.rs: attention_kernels_match_the_fallback reads K/V
 * as transposed views of [B, L, H, D]; the capped-attention inputs take q as
 * a transposed view and K/V as a slice of a cache; the windowed tests read
 * K/V as slices of a larger cache).
 *
 *   q, k, v  non-NULL views of [B,Hq,Lq,D], [B,Hkv,Lk,D], [B,Hkv,Lk,Dv] in
 *            dtype. Strides >= 0 (0 repeats an axis). Each data pointer must
 *            be 16-byte aligned and each stride * sizeof(dtype) a multiple of
 *            16 bytes; k and v row strides below 2^26 bytes.
 *   out      contiguous [B, Hq, Lq, Dv], as for sdpa_forward.
 *   mask_kind / mask  NONE and CAUSAL take no mask (NULL). BOOL: mask->data is
 *            the uint8 [Lq, Lk] matrix with strides (0, 0, Lk). ADDITIVE:
 *            mask->data holds dtype values, element [b, h, i, j] at strides
 *            (stride_b, stride_h, stride_l) and contiguous along j; stride 0
 *            broadcasts (0, h, l for one mask shared by every batch item).
 *   window   0 for none; otherwise >= 1 with SDPA_MASK_CAUSAL, as in
 *            sdpa_forward_windowed.
 * Plans come from sdpa_plan (sdpa_plan_windowed with a window); strides do
 * not change the plan. Other arguments, ownership, errors, scratch and
 * asynchrony as for sdpa_forward.
 */
int sdpa_forward_strided(const sdpa_view_t* q, const sdpa_view_t* k, const sdpa_view_t* v, void* out,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                         int64_t D, int64_t Dv, float scale, int mask_kind,
                         const sdpa_view_t* mask, const void* sinks, int64_t window,
                         int dtype, void* stream);

/*
 * sdpa_forward_noalloc - sdpa_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, validation, kernels and results (the same
 * bits) as sdpa_forward; it calls no hipMalloc, hipFree or other allocating
 * routine. Its scratch (decode partials, packed mask bits: the plan's
 * scratch_bytes) is one fixed array of sdpa_noalloc_scratch_bytes() bytes
 * (16 MiB) per device, held by the library from load until the process ends.
 * A call whose plan needs more returns SDPA_ERR_UNSUPPORTED and enqueues
 * nothing (the decode of B=4, Hq=16, Hkv=2, Lk=65537, D=256 needs 4.3 MB).
 * Every call on one device shares that device's array: calls on that device
 * that overlap in time (on different streams, or graph replays) race with
 * each other; calls ordered on one stream do not. Nothing in the array needs
 * clearing between calls (each call writes what it later reads).
 */
int sdpa_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                         int64_t D, int64_t Dv, float scale,
                         int mask_kind, const uint8_t* mask, const void* sinks,
                         int dtype, void* stream);

/* Size in bytes of sdpa_forward_noalloc's per-device scratch array. */
int64_t sdpa_noalloc_scratch_bytes(void);

/* Message of the last error on the calling thread ("" if none). The pointer
 * stays valid until the thread's next sdpa_* call. */
const char* sdpa_last_error(void);

/* Wait for the devices that used cached scratch (hipDeviceSynchronize), then
 * free every buffer the library holds, replaced ones included. Graphs captured
 * with that scratch must not be replayed afterwards. Returns SDPA_OK or
 * SDPA_ERR_HIP. */
int sdpa_release_workspace(void);

/* ABI version of this header: 5 (2 added the windowed calls, 3 the paged ones,
 * 4 strided views and additive masks, 5 the allocation-free call). */
int sdpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H */
