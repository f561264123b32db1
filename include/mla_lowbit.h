/*
 * mla_lowbit.h -- C ABI of the gfx950 (MI355X) low-bit MLA cache library.
 *
 * What the library computes.  In weight-absorbed MLA decode every query head
 * attends over one shared per-token content latent (d_c = 512) that serves as
 * both key and value, plus one small decoupled RoPE key (d_r = 64) that
 * carries position.  QuantMLA keeps both parts of that cache at low bit width
 * (content INT4 or INT2, RoPE key INT4) and unpacks and dequantizes them inside
 * the attention kernel.  Sources: "QuantMLA: INT4 (and INT2) for both halves of
 * the MLA cache" (TL;DR, flowchart, Key findings), "Hugging Face Releases
 * QuantMLA" (Engineering Trade-offs and Performance), and "QuantMLA's
 * INT4/INT2 KV-cache quantization reports 5x long-context throughput over
 * BF16" (What the low-bit cache changes, for the C4R4 name).
 *
 * Conventions for every call:
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronizes.  Work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL is the null stream) and runs
 *    asynchronously.
 *  - bf16 tensors are IEEE bfloat16 bit patterns, row-major, 16-byte aligned.
 *  - Host-visible arguments are validated before anything is launched; a
 *    failure returns a non-OK status and mla_last_error() describes it.
 *    Device-resident values (slot ids, block-table entries, sequence lengths)
 *    are preconditions: entries outside the page pool are skipped rather than
 *    dereferenced, but the results for the affected rows are then unspecified.
 *  - No exception crosses the ABI.  The library is thread-safe for concurrent
 *    calls on different streams (its only mutable global state is a
 *    thread-local error string and atomic per-device flags recording that a
 *    kernel's LDS size limit has been raised).
 */
#ifndef MLA_LOWBIT_H
#define MLA_LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or count  */
    MLA_ERR_UNSUPPORTED = 2,  /* format or head count this build does not run */
    MLA_ERR_WORKSPACE = 3,    /* workspace smaller than mla_decode_workspace_bytes */
    MLA_ERR_HIP = 4           /* the HIP runtime refused a launch            */
} mla_status_t;

/* Cache encoding.  Supported values:
 *   C4R4 = {4, 64, 4, 64, 512, 64, 64}: content INT4 in groups of 64 channels,
 *          RoPE key INT4 in one group of 64;
 *   C2R4 = {2, 32, 4, 64, 512, 64, 64}: content INT2 in groups of 32 channels,
 *          RoPE key INT4 in one group of 64;
 *   BF16 = {16, 0, 16, 0, 512, 64, 64}: unquantized bf16 rows (the baseline).
 * Quantization is per token and per channel group, asymmetric, with an fp16
 * scale S and an fp16 zero Z: S = fp16((max - min) / (2^b - 1)), Z = fp16(min),
 * code = clamp(round_half_even((x - Z) / S), 0, 2^b - 1) in IEEE fp32 with the
 * stored S and Z (all codes 0 when S == 0), and the dequantized value used by
 * attention is bf16_round_half_even(fma(code, S, Z)). */
typedef struct {
    int32_t c_bits, c_group;   /* content latent: bits (4, 2 or 16), group size */
    int32_t r_bits, r_group;   /* RoPE key: bits (4 or 16), group size          */
    int32_t d_c, d_r;          /* 512, 64                                       */
    int32_t page_size;         /* tokens per page: 64                           */
} mla_format_t;

/* Physical page layout (bytes, little endian), page = page_size tokens.
 * Quantized formats:
 *   [A] content codes   [chunk][token][16 B]: chunk j holds channels
 *       [j*E, (j+1)*E), E = 128 / c_bits; element e of a chunk is in byte
 *       e*b/8 at bit (e*b)%8 (INT4: low nibble first; INT2: low pair first);
 *   [B] content S/Z     [group][token][S16, Z16];
 *   [C] RoPE codes      [chunk][token][16 B], as [A] with d_r and r_bits;
 *   [D] RoPE S/Z        [group][token][S16, Z16].
 * C4R4 page: 16384 + 2048 + 2048 + 256 = 20736 B (324 B per token);
 * C2R4 page:  8192 + 4096 + 2048 + 256 = 14592 B (228 B per token).
 * BF16 page: [token][d_c + d_r] bf16 = 73728 B (1152 B per token).
 * A token's slot is page_id * page_size + offset_in_page. */

/* Bytes per token / per page of `fmt`; 0 if the format is unsupported.
 * Passage: the physical cache layout behind the compression figure ("QuantMLA:
 * INT4 (and INT2) for both halves of the MLA cache", Key findings, systems;
 * "Hugging Face Releases QuantMLA", Engineering Trade-offs and Performance).
 * The pages give no byte breakdown: the layout above is this library's. */
size_t mla_token_bytes(const mla_format_t* fmt);
size_t mla_page_bytes(const mla_format_t* fmt);

/* Quantize and pack n_new new tokens into the paged cache.
 * Passage: the two cache paths, content latent INT4 or INT2 and RoPE key
 * INT4, quantized separately ("QuantMLA: INT4 (and INT2) for both halves of
 * the MLA cache", flowchart and Key findings, bits; "Hugging Face Releases
 * QuantMLA", Engineering Trade-offs and Performance).  Group size, the
 * asymmetric min/max rule and fp16 scale/zero are this library's reading
 * (the pages name bit widths only); the arithmetic is stated with
 * mla_format_t above.
 *   latent_bf16   [n_new, d_c]     content latent rows
 *   rope_bf16     [n_new, d_r]     RoPE key rows (RoPE already applied)
 *   slot_mapping  [n_new] int32    destination slot of each row; a negative
 *                                  slot skips the row; a slot whose page is
 *                                  >= num_pages is skipped
 *   cache         [num_pages * mla_page_bytes(fmt)] bytes, written in place
 * Only the slots named are written (codes, S and Z of every group of the
 * token).  For BF16 the rows are copied unchanged.  n_new == 0 is a no-op.
 * Inputs must be finite with each group's (max - min) / (2^b - 1) and min
 * inside the fp16 range (otherwise S or Z saturate: unspecified codes). */
mla_status_t mla_quant_append(const mla_format_t* fmt,
                              const void* latent_bf16, const void* rope_bf16,
                              const int32_t* slot_mapping, int32_t n_new,
                              void* cache, int64_t num_pages, void* stream);

/* (No passage: the pages describe no kernel.  The split and workspace
 * queries below describe this library's split-KV decode.)
 * A per-sequence split count suited to this shape (from the batch size, the
 * longest sequence and the workgroups the compute units hold at once: two
 * per unit for the quantized formats at 17..32 heads), for callers that want
 * the fixed-split mode; always in [1, 64].  num_splits = 0 (the balanced
 * partition) needs no such choice. */
int32_t mla_decode_num_splits(const mla_format_t* fmt, int32_t batch, int32_t num_heads,
                              int32_t max_seq_len);

/* Workspace bytes mla_decode_lowbit / mla_decode_partial need for this shape
 * (0 for an invalid argument).  num_splits = S >= 1: fp32 partial outputs
 * [batch, S, num_heads, d_c], then fp32 partial log-sum-exps
 * [batch, S, num_heads].  num_splits = 0: the same two arrays over
 * G + batch partial slots, then int32 [batch, 2] (first slot, slot count)
 * per sequence, where G (the balanced partition's workgroups) is the current
 * device's compute units (at most 256 are used; an MI355X has 256) times the
 * workgroups one unit holds: two for the quantized formats at 17..32 rows per
 * sequence, else one (so G = 512 or 256 on an MI355X).  Each array starts
 * 256-byte aligned.  Sizes are for the device current at the call: query them
 * with the device that will run the decode current. */
size_t mla_decode_workspace_bytes(const mla_format_t* fmt, int32_t batch, int32_t num_heads,
                                  int32_t num_splits);

/* Partial slots in that workspace: batch * num_splits, or G + batch for
 * num_splits = 0 (0 for an invalid argument).  num_heads is the rows per
 * sequence, as for mla_decode_workspace_bytes. */
int64_t mla_decode_partial_slots(const mla_format_t* fmt, int32_t batch, int32_t num_heads,
                                 int32_t num_splits);

/* Decode attention over the packed cache, for one query token per sequence.
 * Passage: the native low-bit MLA attention kernel that unpacks and
 * dequantizes the cache inside attention ("QuantMLA: INT4 (and INT2) for both
 * halves of the MLA cache", flowchart and Key findings, systems; "Hugging Face
 * Releases QuantMLA", Engineering Trade-offs and Performance); the content
 * latent is the shared source of keys and values (same wiki note, TL;DR and
 * flowchart), so it is both key and value here, and the learned path
 * transforms are folded into the weights offline (Key findings), so the
 * kernel applies none:
 *   out[b, h, :] = sum_t softmax_t(scale * <q[b,h,:], khat[t,:]>) * khat[t, :d_c]
 *   lse[b, h]    = log sum_t exp(scale * <q[b,h,:], khat[t,:]>)   (natural log)
 * where khat[t] is token t's dequantized [latent | RoPE key] (576 values) and
 * t runs over the first seq_lens[b] tokens of sequence b, found through
 * block_table[b, t / page_size] at offset t % page_size.
 *   q_bf16        [batch, num_heads, d_c + d_r]  absorbed content query then
 *                                                RoPE query, per head
 *   cache         as written by mla_quant_append, num_pages pages
 *   block_table   [batch, max_pages_per_seq] int32 physical page ids; an
 *                 id outside [0, num_pages) within a sequence's length reads
 *                 as a page of zero rows (logit 0, value 0), never out of
 *                 the pool
 *   seq_lens      [batch] int32 tokens per sequence (0 gives out = 0 and
 *                 lse = -inf; values above max_pages_per_seq * page_size are
 *                 clamped to that capacity)
 *   num_heads     1..128
 *   max_pages_per_seq  1..2^24
 *   max_seq_len   host upper bound on seq_lens (sizes the fixed splits)
 *   num_splits    0 = balanced: the batch's pages, in sequence order, are cut
 *                 into min(G, pages) equal shares, one workgroup per share
 *                 (G as for mla_decode_workspace_bytes: one or two per
 *                 compute unit, 256 or 512 on an MI355X), whatever the
 *                 length mix; 1..64 = every
 *                 sequence cut into that many contiguous page ranges.  Either
 *                 way the pieces are merged by log-sum-exp
 *   workspace     >= mla_decode_workspace_bytes(fmt, batch, num_heads,
 *                 num_splits) device bytes, 256-byte aligned; may be NULL
 *                 when num_splits is 1
 *   out_bf16      [batch, num_heads, d_c]
 *   lse_out       [batch, num_heads] fp32, or NULL
 * Results do not depend on how pages are placed in the pool, and are
 * bit-identical from run to run for the same num_splits and seq_lens (the
 * balanced cut depends on every sequence's length). */
mla_status_t mla_decode_lowbit(const mla_format_t* fmt, const void* q_bf16,
                               const void* cache, int64_t num_pages,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                               int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                               void* workspace, size_t workspace_bytes,
                               void* out_bf16, float* lse_out, void* stream);

/* Bytes of device scratch mla_decode_lowbit_noalloc holds on every device the
 * library runs on (128 MiB). */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* mla_decode_lowbit without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of mla_decode_lowbit (same kernels, bitwise the same out and lse); the
 * partial results live in a device array of MLA_NOALLOC_SCRATCH_BYTES that
 * the library holds per device until the process ends.  This call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *  - A shape whose workspace (mla_decode_workspace_bytes(fmt, batch,
 *    num_heads, num_splits)) exceeds MLA_NOALLOC_SCRATCH_BYTES is refused
 *    with MLA_ERR_WORKSPACE before anything is launched.  With the balanced
 *    partition at 128 heads that is about 250 sequences per call.
 *    num_splits = 1 uses no scratch.
 *  - Every call on a device shares that device's array, which keeps the last
 *    call's contents (nothing in it needs to start at zero: the decode
 *    writes every entry the combine reads).  Calls that overlap on one
 *    device (on different streams, or from different threads) race on it:
 *    serialize them.
 *  - The first call on a device looks the array's address up
 *    (hipGetSymbolAddress) with that device current; make that first call
 *    outside graph capture. */
mla_status_t mla_decode_lowbit_noalloc(const mla_format_t* fmt, const void* q_bf16,
                                       const void* cache, int64_t num_pages,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                                       int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                       void* out_bf16, float* lse_out, void* stream);

/* The serving step fused into one call (the pages' cache-pressure serving
 * setting, "QuantMLA's INT4/INT2 KV-cache quantization reports 5x long-context
 * throughput over BF16", Where BF16 caches fall over: every decode step adds
 * one token per sequence to the cache): for every sequence b with
 * seq_lens[b] >= 1, row b of latent_new_bf16 [batch, d_c] and rope_new_bf16
 * [batch, d_r] is quantized and packed into position seq_lens[b] - 1 (page
 * block_table[b, (seq_lens[b] - 1) / page_size], offset (seq_lens[b] - 1) %
 * page_size), then the decode of mla_decode_lowbit runs over all seq_lens[b]
 * tokens, the new one included.  The result (cache bytes, out, lse) is
 * identical to mla_quant_append with those slots followed by
 * mla_decode_lowbit with the same arguments.  The append is done inside the
 * decode kernel by the workgroup that reads the sequence's last page, so the
 * new row makes no separate trip.  A page id outside [0, num_pages) skips
 * the append (as mla_quant_append skips such slots).  Both row pointers must
 * be 16-byte aligned; `cache` is written. */
mla_status_t mla_decode_append_lowbit(const mla_format_t* fmt, const void* latent_new_bf16,
                                      const void* rope_new_bf16, const void* q_bf16, void* cache,
                                      int64_t num_pages, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                      int32_t max_pages_per_seq, int32_t max_seq_len,
                                      float softmax_scale, int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* out_bf16, float* lse_out,
                                      void* stream);

/* The first stage of mla_decode_append_lowbit (append + partial results);
 * mla_decode_combine completes it.  Arguments as mla_decode_append_lowbit
 * and mla_decode_partial. */
mla_status_t mla_decode_append_partial(const mla_format_t* fmt, const void* latent_new_bf16,
                                       const void* rope_new_bf16, const void* q_bf16, void* cache,
                                       int64_t num_pages, const int32_t* block_table,
                                       const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                       int32_t max_pages_per_seq, int32_t max_seq_len,
                                       float softmax_scale, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Multi-token decode (several query tokens per sequence, e.g. multi-token
 * prediction or speculative decoding; no passage: the pages describe one query
 * token, and this extends mla_decode_lowbit causally): the last num_queries tokens of every
 * sequence are queries; query i (0 <= i < num_queries) sits at position
 * seq_lens[b] - num_queries + i and attends to tokens [0, seq_lens[b] -
 * num_queries + 1 + i), i.e. to itself and the tokens before it (their rows
 * are already in the cache).  A query that sees no token gets output 0 and
 * lse -inf.
 *   q_bf16      [batch, num_queries, num_heads, d_c + d_r]
 *   num_queries 1..16
 *   out_bf16    [batch, num_queries, num_heads, d_c]
 *   lse_out     [batch, num_queries, num_heads] fp32, or NULL
 *   workspace   >= mla_decode_workspace_bytes(fmt, batch, num_queries * num_heads,
 *               num_splits) bytes (the rows of a sequence are (query, head) pairs)
 * Other arguments as mla_decode_lowbit.  With num_queries = 1 it is
 * mla_decode_lowbit.  The cache is read once per group of up to 128 rows:
 * num_queries * num_heads <= 128 reads it once. */
mla_status_t mla_decode_multi_lowbit(const mla_format_t* fmt, const void* q_bf16, int32_t num_queries,
                                     const void* cache, int64_t num_pages,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                                     int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                     void* workspace, size_t workspace_bytes, void* out_bf16,
                                     float* lse_out, void* stream);
/* First stage of mla_decode_multi_lowbit; complete it with
 * mla_decode_combine(fmt, batch, num_queries * num_heads, num_splits, ...). */
mla_status_t mla_decode_multi_partial(const mla_format_t* fmt, const void* q_bf16, int32_t num_queries,
                                      const void* cache, int64_t num_pages,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                                      int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of mla_decode_lowbit, for callers that schedule them
 * separately (for example to merge partial results computed elsewhere).
 * No passage: split-KV with a log-sum-exp merge is how this library spreads
 * long contexts over the compute units; the merged result is the softmax
 * of mla_decode_lowbit over all tokens.
 * mla_decode_partial writes, for split s of sequence b, the normalized
 * partial output over that split's pages and its log-sum-exp (-inf for an
 * empty split) into `workspace` (layout of mla_decode_workspace_bytes).
 * mla_decode_combine merges them into out_bf16 / lse_out.  With
 * num_splits = S >= 1, split s of sequence b covers pages [s * P, (s + 1) * P)
 * with P = ceil(ceil(max_seq_len / page_size) / S), the last split running to
 * the end of the sequence.  With num_splits = 0, T = the batch's pages in all
 * and G = min(G of mla_decode_workspace_bytes, T), workgroup w < G takes pages
 * [floor(w * T / G), floor((w + 1) * T / G)) of the concatenation of all
 * sequences' pages (never empty), writes its piece of sequence b to slot
 * w + b, and records each sequence's (first slot, slot count) in the
 * workspace ((0, 0) for an empty sequence).  Both stages
 * must be given the same num_splits, batch and num_heads. */
mla_status_t mla_decode_partial(const mla_format_t* fmt, const void* q_bf16,
                                const void* cache, int64_t num_pages,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                                int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                                void* workspace, size_t workspace_bytes, void* stream);
/* (mla_decode_combine's num_heads is the rows per sequence: num_heads, or
 * num_queries * num_heads after mla_decode_multi_partial; at most 2048.) */
mla_status_t mla_decode_combine(const mla_format_t* fmt, int32_t batch, int32_t num_heads,
                                int32_t num_splits, const void* workspace, size_t workspace_bytes,
                                void* out_bf16, float* lse_out, void* stream);

/* The absorbed projections around the decode (one MLA decode attention
 * step).  The latent is the shared source of every head's key and value
 * ("QuantMLA: INT4 (and INT2) for both halves of the MLA cache", TL;DR and
 * flowchart): head h's key is W_UK[h] c and its value W_UV[h] c, so decode
 * absorbs the query into latent space before attention and applies the value
 * projection to its result after it.  fp32 accumulation, bf16
 * round-to-nearest-even outputs; all pointers device, caller-owned.
 *   mla_absorb_q:    q_out[b, h, 0:512]   = sum_k q_nope[b, h, k] w_uk[h, n, k]
 *                    q_out[b, h, 512:576] = q_pe[b, h, :]
 *     q_nope_bf16 [batch, num_heads, 128], q_pe_bf16 [batch, num_heads, 64],
 *     w_uk_bf16 [num_heads, 512, 128] (n-major), q_out_bf16 [batch, num_heads, 576]
 *     (the q of mla_decode_lowbit)
 *   mla_project_out: out[b, h, j] = sum_c latent[b, h, c] w_uv[h, j, c]
 *     latent_bf16 [batch, num_heads, 512] (the out of mla_decode_lowbit),
 *     w_uv_bf16 [num_heads, 128, 512], out_bf16 [batch, num_heads, 128]
 * num_heads 1..1024; q_nope, w_uk, q_out, latent, w_uv 16-byte aligned. */
mla_status_t mla_absorb_q(const void* q_nope_bf16, const void* q_pe_bf16, const void* w_uk_bf16,
                          int32_t batch, int32_t num_heads, void* q_out_bf16, void* stream);
mla_status_t mla_project_out(const void* latent_bf16, const void* w_uv_bf16, int32_t batch,
                             int32_t num_heads, void* out_bf16, void* stream);

/* Description of the most recent non-OK status returned on this thread. */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_LOWBIT_H */
