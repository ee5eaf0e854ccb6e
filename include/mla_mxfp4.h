/*
 * mla_mxfp4.h -- C ABI of libmla_mxfp4.so: MXFP4-KV absorbed-MLA decode for
 * AMD Instinct MI355X (gfx950), with fp8-KV and bf16-KV sibling decodes on
 * the same plan (mla_decode_fp8, mla_decode_bf16).
 *
 * The operation (kernelindex.com "amd-mixed-mla" submission pages):
 *   For each sequence b (one query token) and head h in 0..15,
 *     out[b,h,:] = sum_t softmax_t(sm_scale * q[b,h,:] . K[t,:]) * V[t,:]
 *   over the tokens t of b, where K[t,:] (576 values) is the MXFP4-decoded
 *   latent+rope row and V[t,:] = K[t,0:512]. Definition: page
 *   "kernelbot-amd-mixed-mla-676098", _naive_fallback; shapes and the cache
 *   layout: page "kernelbot-amd-mixed-mla-608791", constants block and
 *   stage-1 kernel.
 *
 * Data layouts (all row-major and contiguous):
 *   q         bf16  [B, 16, 576]   device, 16-byte aligned
 *   kv_packed uint8 [T, 288]       device, 16-byte aligned. Element j of a
 *             token is the low nibble (j even) or high nibble (j odd) of byte
 *             j/2, an OCP e2m1 code ("kernelbot-amd-mixed-mla-608791",
 *             kFp4Lut and the stage-1 tile fill).
 *   kv_scale  uint8 [T, 18]        device, any byte alignment. E8M0 byte e scales
 *             elements 32k..32k+31 by 2^(e-127); e = 255 is NaN
 *             ("kernelbot-amd-mixed-mla-608791", e8m0_to_float).
 *   kv_indptr int32 [B+1]          non-decreasing token offsets of the
 *             sequences (page size 1, as on the 608791 page).
 *   out       bf16  [B, 16, 512]   device, 16-byte aligned; written, never
 *             read. A sequence with no tokens gets zeros.
 * The decode is exact for E8M0 bytes 2..252 (every decoded element is then a
 * normal bf16 value); bytes 253/254 can overflow bf16 and give inf/NaN.
 *
 * Ownership: the caller allocates every buffer (q, cache, out, workspace) and
 * the library allocates no device memory. mla_decode_mxfp4 never blocks the
 * host and only enqueues kernels on the given stream, so it may be recorded
 * in a HIP graph. All pointers stay owned by the caller.
 *
 * Errors: every call returns an int status (MLA_OK = 0 or a negative code);
 * mla_last_error() gives a message for the calling thread's last failure.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = default stream).
 */
#ifndef MLA_MXFP4_H
#define MLA_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem constants ("kernelbot-amd-mixed-mla-608791", constants block). */
#define MLA_NUM_HEADS 16
#define MLA_QK_DIM 576
#define MLA_V_DIM 512
#define MLA_SCALE_BLOCK 32
#define MLA_PACKED_BYTES 288
#define MLA_SCALES_PER_TOKEN 18
/* The 24-scale layout (page "kernelbot-amd-mixed-mla-717900", mxfp4 layout
 * comment block): 24 E8M0 bytes per token, byte k scaling elements
 * 24k .. 24k+23. */
#define MLA_SCALE_BLOCK_24 24
#define MLA_SCALES_PER_TOKEN_24 24

/* Planner constants: workgroups per compute unit, slot rounding, minimum
 * slot length in tokens, and the fixed work of one item (its Q, its first
 * tile, the merge and stores) in tokens of streaming. The plan rule is
 * stated at mla_plan below. */
#define MLA_PLAN_WG_PER_CU 1
#define MLA_PLAN_CHUNK_ALIGN 128
#define MLA_PLAN_MIN_CHUNK 256
#define MLA_PLAN_ITEM_COST 512
#define MLA_PLAN_MAGIC 0x4D4C4134
#define MLA_PLAN_VERSION 1
#define MLA_PLAN_HEADER_WORDS 16

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID -1      /* bad argument: null/misaligned pointer, bad indptr, batch < 0, non-finite sm_scale, ... */
#define MLA_ERR_WORKSPACE -2    /* workspace smaller than the plan needs */
#define MLA_ERR_HIP -3          /* a HIP runtime call or kernel launch failed */
#define MLA_ERR_DEVICE -4       /* the current device is not gfx950 */
#define MLA_ERR_NOT_PLANNED -5  /* workspace was never passed to mla_plan, or was released */

/* Human-readable name of a status code (static string). */
const char* mla_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* mla_last_error(void);

/* Number of compute units of the current HIP device (queried once per
 * device). Returns MLA_ERR_DEVICE if the device is not gfx950. */
int mla_device_num_cus(int32_t* num_cus);

/* Upper bound, in bytes, on the workspace a plan for `batch` sequences with
 * `total_kv` tokens needs on a device with `num_cus` compute units
 * (num_cus <= 0: query the current device). The workspace holds the plan
 * words followed by the split-K partials (float32 LSE [P,16] and normalised
 * float32 outputs [P,16,512]). MLA_ERR_INVALID for batch < 0, total_kv
 * outside [0, 2^31), or sizes whose worst-case plan would start its
 * partial outputs past the int32 byte offsets a plan stores (tens of
 * millions of sequences). */
int mla_workspace_bytes(int32_t batch, int64_t total_kv, int32_t num_cus, size_t* bytes);

/* Build the work list for a host copy of kv_indptr ([batch+1]) and copy it
 * into `workspace` (device memory, 256-byte aligned, `workspace_bytes` long)
 * on `stream`; returns after the copy has completed. The plan stays valid
 * for decode calls on the same kv_indptr values.
 *
 * Plan rule (the pages leave the split policy open; page
 * "kernelbot-amd-mixed-mla-608791", host metadata builder, gives the role of
 * the work list and per-batch partial index): with T = kv_indptr[B] -
 * kv_indptr[0] tokens and G = num_cus * MLA_PLAN_WG_PER_CU workgroups,
 * c0 = max(MLA_PLAN_MIN_CHUNK, round_up(ceil(T/G), MLA_PLAN_CHUNK_ALIGN)) is
 * the equal-token slot. When c0 > MLA_PLAN_ITEM_COST, a sequence of length
 * 0 < n < c0 is short: it shares its slot with others and each of its items
 * adds fixed work. The sequences are laid end to end on a weighted line, a
 * short one taking MLA_PLAN_ITEM_COST units and then its n tokens, a long
 * one its tokens only (so with no short sequence the line is the token
 * stream); Wt is the line's length, chunk = max(MLA_PLAN_MIN_CHUNK,
 * round_up(ceil(Wt/G), MLA_PLAN_CHUNK_ALIGN)), and slot s owns the units
 * [s*chunk, (s+1)*chunk). Each slot's tokens are cut at sequence boundaries
 * into items; an item covering a whole sequence writes its output directly,
 * any other item writes a partial (acc, LSE) merged afterwards by the
 * reduce kernel.
 *
 * Errors: MLA_ERR_INVALID for batch < 0, a null indptr (batch > 0),
 * indptr[0] < 0, decreasing offsets, more than 2^31-1 tokens or a null or
 * misaligned workspace; MLA_ERR_WORKSPACE if workspace_bytes is too small. */
int mla_plan(const int32_t* kv_indptr_host, int32_t batch,
             void* workspace, size_t workspace_bytes, void* stream);

/* mla_plan with an explicit compute-unit count (num_cus <= 0: query the
 * device). Used to test that results do not depend on the split. */
int mla_plan_cus(const int32_t* kv_indptr_host, int32_t batch, int32_t num_cus,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Build the work list on the GPU from a device copy of kv_indptr
 * ([batch+1] int32, 4-byte aligned): one kernel enqueued on `stream`, no
 * host synchronisation and no host read of the offsets, so plan + decode can
 * be recorded in one HIP graph and replayed while kv_indptr changes in place
 * (page "kernelbot-amd-mixed-mla-717900" records both decode stages in a
 * graph; page "kernelbot-amd-mixed-mla-608791", host metadata builder, gives
 * the work list this fills).
 *
 * Same plan rule and the same items, partial indices and reduce entries as
 * mla_plan for the same offsets; only the section offsets differ, since the
 * words are laid out for the bounds: every replay must keep
 * kv_indptr[batch] - kv_indptr[0] <= max_total_kv, and the workspace must
 * hold mla_workspace_bytes(batch, max_total_kv, num_cus) bytes.
 * num_cus <= 0: the current device's count.
 *
 * Errors returned (nothing enqueued): MLA_ERR_INVALID (batch < 0,
 * max_total_kv outside [0, 2^31), null or misaligned kv_indptr or
 * workspace), MLA_ERR_WORKSPACE, MLA_ERR_DEVICE, MLA_ERR_HIP. Offsets that
 * are invalid on the device (decreasing, kv_indptr[0] < 0, more than
 * max_total_kv tokens) give an empty plan: header magic 0, no slots and no
 * reduce entries, so the decode then writes nothing. */
int mla_plan_device(const int32_t* kv_indptr_dev, int32_t batch, int64_t max_total_kv,
                    int32_t num_cus, void* workspace, size_t workspace_bytes, void* stream);

/* Forget the plan registered for `workspace` (a host-side record; the
 * device memory is not touched). Call it before the workspace memory is
 * freed or reused: a decode on a released workspace returns
 * MLA_ERR_NOT_PLANNED until it is planned again. The registry is keyed by
 * address, so a workspace freed without release and reallocated at the
 * same address would otherwise still find the old record; the decode
 * kernels then follow the words in the workspace only if its header holds
 * the plan magic and version (anything else leaves `out` untouched), but
 * an old plan left intact in the memory cannot be told from a fresh one.
 * Returns MLA_OK, or MLA_ERR_NOT_PLANNED if no plan was registered.
 * Thread-safe; needs no GPU. */
int mla_plan_release(void* workspace);

/* Host-only planner: write the plan words for `num_cus` compute units into
 * `words` (host, `capacity_words` int32 entries). On success *num_words is
 * the word count and *workspace_bytes the workspace size the plan needs.
 * Touches no GPU. MLA_ERR_WORKSPACE if capacity_words is too small (then
 * *num_words still reports the needed count). */
int mla_plan_host(const int32_t* kv_indptr_host, int32_t batch, int32_t num_cus,
                  int32_t* words, size_t capacity_words, size_t* num_words,
                  size_t* workspace_bytes);

/* Run the decode planned into `workspace` by mla_plan or mla_plan_device
 * (same kv_indptr values). Enqueues the split-K decode kernel and, when some sequence is
 * split or empty, the LSE-weighted reduce kernel on `stream`; never
 * synchronises. kv_indptr is the device copy of the offsets the plan was
 * built from; the kernels use it to bound every item to its sequence.
 * sm_scale is the softmax scale (1/sqrt(576) for this model); any finite
 * value (zero gives the plain mean of V, a negative scale favours the
 * lowest scores, as the definition does).
 *
 * The kernels only follow plan words whose header holds MLA_PLAN_MAGIC and
 * MLA_PLAN_VERSION; a workspace whose header does not (cleared or
 * overwritten after planning, or an empty device plan) leaves `out`
 * untouched.
 *
 * Errors (nothing is enqueued): MLA_ERR_NOT_PLANNED (checked first, without
 * any HIP call), MLA_ERR_INVALID (null or misaligned pointer, non-finite
 * sm_scale), MLA_ERR_DEVICE, MLA_ERR_HIP (launch failure). Faults inside
 * the kernels surface as HIP errors on the stream. */
int mla_decode_mxfp4(const void* q, const void* kv_packed, const void* kv_scale,
                     const int32_t* kv_indptr, void* out, float sm_scale,
                     void* workspace, void* stream);

/* mla_decode_mxfp4 for callers that cannot allocate device memory (code
 * recorded into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument and no allocation of any kind. The plan
 * words and split-K partials live in a static device array of the library
 * (20 MiB, held by every GPU the library runs on until the process ends);
 * the plan is built on the GPU from the device copy of kv_indptr ([batch+1]
 * int32, 4-byte aligned), by the same rule and with the same items as
 * mla_plan, so the output equals mla_decode_mxfp4's on a plan of the same
 * offsets. q, kv_packed, kv_scale, out, sm_scale and stream as for
 * mla_decode_mxfp4; kv_indptr may change in place between calls (up to
 * 2^31 - 1 tokens). The array is shared by every call on a GPU and keeps
 * the last call's contents: calls that overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller.
 *
 * Errors (nothing enqueued): MLA_ERR_INVALID (batch < 0, non-finite
 * sm_scale, null or misaligned pointer), MLA_ERR_WORKSPACE when the plan
 * and partials of `batch` sequences exceed the static array (more than
 * 129,885 sequences on a 256-CU device), MLA_ERR_DEVICE, MLA_ERR_HIP. */
int mla_decode_mxfp4_noalloc(const void* q, const void* kv_packed, const void* kv_scale,
                             const int32_t* kv_indptr, int32_t batch, void* out, float sm_scale,
                             void* stream);

/* The same decode over the 24-scale MXFP4 layout of page
 * "kernelbot-amd-mixed-mla-717900" (mxfp4 layout comment block and the
 * stage-1 loads of its Triton decode): kv_packed uint8 [T, 288] as for
 * mla_decode_mxfp4 (element 2j the low nibble of byte j, e2m1 codes), and
 * kv_scale uint8 [T, 24] (device, 8-byte aligned) whose byte k scales
 * elements 24k .. 24k+23 (packed bytes 12k .. 12k+11) by 2^(byte-127); 255
 * is NaN. V is again the first 512 decoded elements. The plan, workspace,
 * q, kv_indptr, out, sm_scale, stream, ownership and error codes are those
 * of mla_decode_mxfp4 (one plan serves every cache format), plus
 * MLA_ERR_INVALID for a kv_scale that is not 8-byte aligned. The decoded
 * elements are exact for scale bytes 2..252, as for the 18-scale layout. */
int mla_decode_mxfp4_24(const void* q, const void* kv_packed, const void* kv_scale,
                        const int32_t* kv_indptr, void* out, float sm_scale,
                        void* workspace, void* stream);

/* The same decode over a cache whose rows are listed per token (page size
 * 1): sequence b reads rows kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] of
 * the row pools kv_packed (uint8 [R, 288], 16-byte aligned) and kv_scale
 * (uint8 [R, 18], 2-byte aligned) -- the kv_indices / page_size = 1 layout
 * of the decode call on page "kernelbot-amd-mixed-mla-676098"
 * (_aiter_mla_decode). kv_indices is int32 [kv_indptr[B]] on the device
 * (4-byte aligned); entries before kv_indptr[0] are not read. Rows may be
 * shared between sequences and appear in any order. Every index must lie
 * in [0, R) and R * 288 must stay below 2^32 (offsets are 32-bit): the
 * library cannot check this without reading the indices, so the caller
 * guarantees it (the Python binding checks it). The plan is the one of
 * mla_plan / mla_plan_device over the same kv_indptr; everything else as for
 * mla_decode_mxfp4. */
int mla_decode_mxfp4_paged(const void* q, const void* kv_packed, const void* kv_scale,
                           const int32_t* kv_indices, const int32_t* kv_indptr, void* out,
                           float sm_scale, void* workspace, void* stream);

/* The same decode over an fp8 KV cache: kv_fp8 is uint8 [T, 576] (device,
 * 16-byte aligned), each byte an OCP FP8 E4M3 code (the MI355X fp8 type:
 * 4 exponent bits with bias 7, 3 mantissa bits, largest finite value 448,
 * codes 0x7F/0xFF NaN), and kv_scale points to ONE float32 on the device
 * (4-byte aligned) that scales the whole tensor: K[t,j] = e4m3(kv_fp8[t,j]) *
 * kv_scale[0], V[t,:] = K[t,0:512]. This is the fp8 cache of page
 * "kernelbot-amd-mixed-mla-676098" (_aiter_mla_decode: kv_fp8, kv_scale =
 * kv_data["fp8"]). q, kv_indptr, out, sm_scale, the workspace (planned by
 * mla_plan / mla_plan_device: the plan does not depend on the cache
 * format), the stream, ownership and the error codes are those of
 * mla_decode_mxfp4. */
int mla_decode_fp8(const void* q, const void* kv_fp8, const float* kv_scale,
                   const int32_t* kv_indptr, void* out, float sm_scale,
                   void* workspace, void* stream);

/* The same decode over a bf16 KV cache: kv_bf16 is bfloat16 [T, 576]
 * (device, 16-byte aligned), K[t,:] = row t, V[t,:] = K[t,0:512] (page
 * "kernelbot-amd-mixed-mla-676098", _naive_fallback reads kv_data["bf16"]).
 * Everything else as for mla_decode_mxfp4. */
int mla_decode_bf16(const void* q, const void* kv_bf16, const int32_t* kv_indptr,
                    void* out, float sm_scale, void* workspace, void* stream);

/* mla_decode_fp8 and mla_decode_bf16 over per-token row lists: sequence b
 * reads rows kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] of the row pool
 * (fp8: uint8 [R, 576]; bf16: bfloat16 [R, 576]; 16-byte aligned), with the
 * rules of mla_decode_mxfp4_paged: kv_indices int32 on the device, 4-byte
 * aligned, every index in [0, R), R * row bytes below 2^32, checked by the
 * caller. */
int mla_decode_fp8_paged(const void* q, const void* kv_fp8, const float* kv_scale,
                         const int32_t* kv_indices, const int32_t* kv_indptr, void* out,
                         float sm_scale, void* workspace, void* stream);
int mla_decode_bf16_paged(const void* q, const void* kv_bf16, const int32_t* kv_indices,
                          const int32_t* kv_indptr, void* out, float sm_scale,
                          void* workspace, void* stream);

/* The three decodes over contiguous rows that sequences may share: sequence
 * b reads rows kv_start[b] .. kv_start[b] + (kv_indptr[b+1] - kv_indptr[b])
 * - 1 of the cache (kv_start: int32 [B] on the device, 4-byte aligned),
 * while kv_indptr (the offsets the plan was built from) only gives the
 * lengths and the order of work. Several query entries can then attend the
 * same rows. Page "kernelbot-amd-mixed-mla-676098" runs q_seq_len query
 * tokens per sequence in its Triton decode, query token i over the whole
 * KV range of sequence i / q_seq_len. A 128-head query (the H = 128
 * configuration named on the same page) is eight 16-head groups over the
 * same rows. Each entry is a full 16-head decode and reads its rows
 * itself. The caller guarantees that every row read lies inside the cache
 * (the Python binding checks it). Pools, q, out and everything else as
 * for the plain decodes of each format; MLA_ERR_INVALID for a null or
 * misaligned kv_start. */
int mla_decode_mxfp4_starts(const void* q, const void* kv_packed, const void* kv_scale,
                            const int32_t* kv_start, const int32_t* kv_indptr, void* out,
                            float sm_scale, void* workspace, void* stream);
int mla_decode_fp8_starts(const void* q, const void* kv_fp8, const float* kv_scale,
                          const int32_t* kv_start, const int32_t* kv_indptr, void* out,
                          float sm_scale, void* workspace, void* stream);
int mla_decode_bf16_starts(const void* q, const void* kv_bf16, const int32_t* kv_start,
                           const int32_t* kv_indptr, void* out, float sm_scale, void* workspace,
                           void* stream);

/* The three decodes over a page table (page "kernelbot-amd-mixed-mla-676098",
 * _aiter_mla_decode, passes kv_indptr, kv_indices, kv_last_page_len and
 * page_size to its decode; page_size is 1 there). Sequence b owns pages
 * page_indices[page_indptr[b] .. page_indptr[b+1]-1] (int32, device, 4-byte
 * aligned, both), each a run of page_size consecutive rows of the row pools
 * (MXFP4: kv_packed [R, 288] and kv_scale [R, 18], 2-byte aligned; fp8:
 * uint8 [R, 576]; bf16: bfloat16 [R, 576]). Token t of the sequence (t from
 * 0) is pool row page_indices[page_indptr[b] + t / page_size] * page_size +
 * t % page_size. kv_indptr is the device copy of the token offsets the plan
 * was built from: sequence b has kv_indptr[b+1] - kv_indptr[b] tokens, that
 * is (pages - 1) * page_size plus the valid rows of its last page
 * (kv_last_page_len, 1..page_size). page_size >= 1 (any value; page_size 1
 * with page_indptr = kv_indptr is the row list of the *_paged calls).
 * The caller guarantees that the page counts match the token counts and
 * that every row read lies in [0, R) with R * row bytes below 2^32 (the
 * Python binding checks both); the library cannot check them without
 * reading the arrays. Errors: those of the *_paged calls, plus
 * MLA_ERR_INVALID for page_size < 1 or a null or misaligned page_indptr
 * or page_indices. */
int mla_decode_mxfp4_page_table(const void* q, const void* kv_packed, const void* kv_scale,
                                const int32_t* page_indices, const int32_t* page_indptr,
                                int32_t page_size, const int32_t* kv_indptr, void* out,
                                float sm_scale, void* workspace, void* stream);
int mla_decode_fp8_page_table(const void* q, const void* kv_fp8, const float* kv_scale,
                              const int32_t* page_indices, const int32_t* page_indptr,
                              int32_t page_size, const int32_t* kv_indptr, void* out,
                              float sm_scale, void* workspace, void* stream);
int mla_decode_bf16_page_table(const void* q, const void* kv_bf16, const int32_t* page_indices,
                               const int32_t* page_indptr, int32_t page_size,
                               const int32_t* kv_indptr, void* out, float sm_scale,
                               void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_MXFP4_H */
