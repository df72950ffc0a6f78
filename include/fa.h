/*
 * fa.h — C ABI of libfa.so: causal grouped-query flash attention on AMD Instinct MI355X
 * (gfx950), with f16, bf16 or 4-bit block-quantized (q4_0) K/V.
 *
 * What every call computes (the fused scaled-dot-product attention forward pass that the
 * mlxcel PR #2306 "defer SDPA accumulator rescale, stage Q once per block" optimises and
 * that the mi210-llm-stack guide "Build FlashAttention (CK backend) on gfx90a" verifies
 * against torch's scaled_dot_product_attention):
 *
 *     O[b,i,h,:] = sum_j softmax_j(scale * Q[b,i,h,:] . K[b,j,g,:]) * V[b,j,g,:]
 *
 * over the keys j that query i may see, with g = h / (Hq / Hkv) (consecutive grouping of
 * "GQA 32/8"). When causal != 0, query i sits at absolute position i + causal_offset and
 * sees key j iff j <= i + causal_offset ("maskless" causal: the mask comes from indices; a
 * chunk of Sq queries placed at the end of Sk keys uses causal_offset = Sk - Sq). A query
 * that sees no key gets a zero output row.
 *
 * Layouts (all contiguous, row-major, no padding):
 *   Q, O : [B, Sq, Hq, D]  elements of the Q type
 *   K, V : [B, Sk, Hkv, D] elements of the K/V type, or for a q4_0 cache
 *          [B, Sk, Hkv, D/32] blocks of 18 bytes (each tensor by its own type when
 *          kv_dtype is mixed)
 * The Q/O type is bf16 when kv_dtype is FA_KV_BF16 and f16 otherwise (f16, q4_0 and mixed
 * caches).
 *
 * q4_0 block (the KV-cache type "-ctk q4_0 -ctv q4_0" of the mi210-llm-stack page
 * "FlashAttention on gfx90a"; the page names it but does not define it, so this is the
 * common GGML arrangement): 32 consecutive head-dim elements, stored as a little-endian f16
 * scale d followed by 16 bytes; byte t holds the 4-bit code c of element t in its low nibble
 * and of element t+16 in its high nibble. Element value: (c - 8) * d.
 *
 * Ownership: every pointer is caller-owned device memory (hipMalloc or a framework's
 * allocator); the library allocates nothing, keeps no device state and never frees.
 * Calls are asynchronous on `stream` (0 = the null stream). A return of FA_OK means the
 * work was enqueued; all argument checks happen before any HIP call, so an error return
 * means nothing was launched. No C++ exception crosses this interface. The library never
 * falls back to a slower path: an unsupported combination is an error.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t *fa_stream_t;

enum fa_kv_dtype {
    FA_KV_F16 = 0,       /* K/V f16,  Q/O f16  */
    FA_KV_BF16 = 1,      /* K/V bf16, Q/O bf16 */
    FA_KV_Q4_0 = 2,      /* K/V q4_0, Q/O f16  */
    /* mixed caches (mi210-llm-stack, "FlashAttention on gfx90a", sets the K and V cache
       types with separate flags, -ctk and -ctv) */
    FA_KV_F16_Q4_0 = 3,  /* K f16, V q4_0, Q/O f16 */
    FA_KV_Q4_0_F16 = 4,  /* K q4_0, V f16, Q/O f16 */
};

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,         /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,        /* negative size, Hq % Hkv != 0, or an index that overflows */
    FA_ERR_DTYPE = -3,        /* kv_dtype (x_dtype) not one of enum fa_kv_dtype (fa_src_dtype) */
    FA_ERR_UNSUPPORTED = -4,  /* valid but not built: D not in {64, 128}; decode rows > 16 */
    FA_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
    FA_ERR_ALIGN = -6,        /* Q/O/K/V not 16-byte aligned (a q4_0 K or V: 4-byte aligned) */
    FA_ERR_HIP = -7,          /* the HIP runtime reported an error at launch */
    FA_ERR_VALUE = -8,        /* scale not finite and > 0 */
    FA_ERR_TOO_LARGE = -9,    /* fa_decode_noalloc: more scratch than FA_NOALLOC_SCRATCH_BYTES */
};

/*
 * Chunked / causal prefill: any Sq, Sk. One MFMA kernel launch.
 *   q, o      device pointers, [B, Sq, Hq, D]
 *   k, v      device pointers, [B, Sk, Hkv, D] (q4_0: [B, Sk, Hkv, D/32] blocks)
 *   B, Hq, Hkv, Sq, Sk, D   sizes; Hq % Hkv == 0; D in {64, 128}; B, Sq, Sk >= 0
 *   causal    0 = every query sees every key; else the rule above with causal_offset
 *   scale     softmax scale, finite and > 0 (typically 1/sqrt(D))
 *   kv_dtype  enum fa_kv_dtype
 * Per row the kernel keeps its O accumulators and sum in the softmax frame it was last
 * rescaled to and rescales only when a block maximum exceeds that frame by more than 10
 * (natural-log units), as the mlxcel PR describes; Q is staged once per workgroup.
 */
int fa_prefill(const void *q, const void *k, const void *v, void *o,
               int B, int Hq, int Hkv, int Sq, int Sk, int D,
               int causal, int64_t causal_offset, float scale, int kv_dtype,
               fa_stream_t stream);

/*
 * Causal prefill with the work balanced across workgroups. In a causal chunk the later query
 * blocks see more keys, so the workgroups that own them hold more 64-key tiles and the call
 * waits for them (at 2048 queries against 2048 keys the tiles per workgroup run from 1 to
 * 32). Where the tile count grows with the query block, blocks q and n-1-q together hold about
 * twice the average, so fa_prefill_split pairs them: a unit (b, KV head, head chunk, 64-row
 * query block) of block q >= q_split holds more than `cap` tiles (cap = the average tiles per
 * unit plus a small bias, q_split >= n/2) and runs only its first cap tiles; the workgroup of
 * its mirror block n-1-q, a light unit, runs the remaining tiles after its own unit. The grid
 * stays one workgroup per unit. The later of a split unit's two parts to finish merges them
 * (log-sum-exp of the two partial softmax states) and writes the unit's rows. No workgroup
 * waits for another. Pairing applies up to 256 units (one workgroup per CU); with more, the
 * workgroups run in several rounds whose dispatch onto the CUs that free up already evens the
 * load, and nothing is paired.
 * With at most 128 units, half the 256 CUs (a short chunk of queries against many keys, or a
 * small batch), most CUs would idle while each unit's workgroup runs all of its tiles, so
 * instead every unit's tiles are cut into runs of at least 4 tiles, as many runs per unit as
 * fill the 256 CUs once (at most 64), each run writes its partial softmax state to the
 * workspace, and a second kernel merges the runs of every row (the same log-sum-exp combine).
 * The arrival counters are not used then.
 * A cache with a q4_0 tensor whose KV heads each have 16 or more 64-row query blocks (for GQA
 * 4, 1024 or more queries) is first widened to f16 in the workspace (the q4_0 tensor or both,
 * with the routine fa_dequant_q4_0 runs), and the split runs on the copies: the in-kernel
 * dequantization is repeated by every query block that reads a tile, one pass over the cache
 * costs less there. The output bits are those of the fused kernel.
 * Arguments as fa_prefill, plus the caller-owned workspace:
 *   workspace   >= fa_prefill_workspace_bytes(...) bytes, 16-byte aligned. Its first 4096
 *               bytes are arrival counters that must be zero before the first call that uses
 *               the workspace (allocate it zero-filled, or clear it once); every call returns
 *               them to zero when it completes, so the workspace can be reused for any later
 *               call without clearing. The rest holds the split units' partial rows, then any
 *               f16 copies of the cache (B * Sk * Hkv * D * 2 bytes each). Non-zero counter
 *               bytes give wrong output rows, never an access outside the workspace.
 *               Calls that share a workspace must be ordered on one stream.
 * Contiguous caches only. A q4_0 tensor at D = 64 splits only through its f16 copy; non-causal
 * calls only by the key split. For shapes with nothing to split and no copy
 * (fa_prefill_workspace_bytes returns 0) the call is fa_prefill and the workspace may be NULL.
 * Errors as fa_prefill, plus FA_ERR_WORKSPACE.
 */
size_t fa_prefill_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                                  int64_t causal_offset, int kv_dtype);
int fa_prefill_split(const void *q, const void *k, const void *v, void *o,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     int causal, int64_t causal_offset, float scale, int kv_dtype,
                     void *workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * Split-K decode. The pages give decode only as model-level token rates (mi210-llm-stack,
 * "FlashAttention on gfx90a", "The Problem": FA on against FA off); the split-K organisation
 * with a log-sum-exp merge is this library's design for the memory-bound one-token step, not
 * a passage of the pages. What each row computes is the same attention as fa_prefill.
 *
 * Bytes of workspace fa_decode needs for these sizes (0 when nothing is needed). Hkv is an
 * argument because the kernel choice, and with it the split count, depends on it.
 * The workspace holds one partial (running max, sum, unnormalised output row) per query
 * row and key split; it is scratch between the split kernel and the merge kernel of one
 * call and need not be initialised.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D);

/*
 * Decode: few query rows per KV head (Sq * Hq / Hkv <= 16), long Sk. The keys are cut
 * into splits that run in parallel; each split writes a partial softmax state to the
 * workspace and a second kernel merges the splits with a log-sum-exp combine. Arguments
 * as fa_prefill plus the caller-owned workspace (>= fa_decode_workspace_bytes(...) bytes,
 * 16-byte aligned). Calls that share a workspace must be ordered on one stream.
 */
int fa_decode(const void *q, const void *k, const void *v, void *o,
              int B, int Hq, int Hkv, int Sq, int Sk, int D,
              int causal, int64_t causal_offset, float scale, int kv_dtype,
              void *workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, kernels, results and
 * errors as fa_decode, without the workspace: the split partials go to a fixed scratch array
 * of FA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the process ends.
 * The call itself allocates nothing (no hipMalloc, no allocating library routine); its first
 * call on a device looks up that device's copy of the array (the device that is current must
 * be the stream's). Calls that need more scratch than the maximum (fa_decode_workspace_bytes
 * of the call above it; 4.3 MB at 4 sequences x 32768 q4_0 keys, GQA 32/8, D = 128) return
 * FA_ERR_TOO_LARGE before any HIP call. Every call on one GPU shares that GPU's array (it keeps
 * the last call's partials; nothing in it needs to start at zero), so calls that may overlap
 * on one GPU (different streams, or different threads without ordering) race and give wrong
 * output: order them on one stream.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o,
                      int B, int Hq, int Hkv, int Sq, int Sk, int D,
                      int causal, int64_t causal_offset, float scale, int kv_dtype,
                      fa_stream_t stream);

/*
 * Split-K decode over paged K/V caches (a batch of sequences of different lengths, as a
 * serving loop keeps them). K and V are n_pages pages of 64 keys each, [n_pages, 64, Hkv, D]
 * (q4_0: [n_pages, 64, Hkv, D/32] blocks of 18 bytes), shared by all sequences; sequence b has
 * seq_lens[b] keys (clamped to [0, max_pages * 64]) and its key j is key j % 64 of page
 * block_table[b * max_pages + j / 64]. Its Sq queries are its last Sq positions: with causal,
 * query i (at position seq_lens[b] - Sq + i) sees keys j <= seq_lens[b] - Sq + i; otherwise
 * all seq_lens[b] keys.
 *   q, o          device pointers, [B, Sq, Hq, D], as fa_decode
 *   block_table   device int32 [B, max_pages]; seq_lens device int32 [B]; 4-byte aligned.
 *                 Entries outside [0, n_pages) are clamped into it (wrong output, never an
 *                 access outside the pages).
 *   workspace     >= fa_decode_workspace_bytes(B, Hq, Hkv, Sq, max_pages * 64, D) bytes.
 * Other arguments, limits, errors and asynchrony as fa_decode.
 */
int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, void *o,
                    const int32_t *block_table, const int32_t *seq_lens, int B, int Hq,
                    int Hkv, int Sq, int D, int max_pages, int n_pages, int causal, float scale,
                    int kv_dtype, void *workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * Chunked prefill over paged K/V caches: a batch of sequences of different lengths, each
 * appending a chunk of its own length, as a serving loop runs them. Pages, block_table,
 * seq_lens and their clamping as fa_decode_paged. Sequence b has q_lens[b] new queries
 * (clamped to [0, Sq]; q_lens NULL means Sq in every sequence) in rows [0, q_lens[b]) of
 * Q[b] and O[b]; they are its last q_lens[b] positions: with causal, row i (at position
 * seq_lens[b] - q_lens[b] + i) sees keys j <= seq_lens[b] - q_lens[b] + i, else all
 * seq_lens[b] keys. Rows i >= q_lens[b] of O are not written.
 *   q, o          device pointers, [B, Sq, Hq, D], as fa_prefill
 *   block_table   device int32 [B, max_pages]; seq_lens, q_lens device int32 [B]; 4-byte
 *                 aligned
 *   max_pages     at most 4096 (a sequence's page numbers are held in LDS), else
 *                 FA_ERR_UNSUPPORTED
 * Other arguments, limits, errors and asynchrony as fa_prefill.
 */
int fa_prefill_paged(const void *q, const void *k_pages, const void *v_pages, void *o,
                     const int32_t *block_table, const int32_t *seq_lens, const int32_t *q_lens,
                     int B, int Hq, int Hkv, int Sq, int D, int max_pages, int n_pages,
                     int causal, float scale, int kv_dtype, fa_stream_t stream);

/*
 * Standard (non-flash) attention, the comparison arm of the mi210-llm-stack page
 * "FlashAttention on gfx90a" ("Three Patching Approaches", Approach C; "The V Dequantization
 * Gap"): that page's fast path is the non-FA one, with K dequantized before use and V to be
 * dequantized the same way. Here, per (b, KV head): a q4_0 K or V is dequantized to f16 (the
 * routine of fa_dequant_q4_0); S = scale * Q K^T is written to the workspace in f32 for every
 * tile holding a visible pair; a row softmax over the visible keys writes P = exp(S - max) /
 * sum in the Q type; O = P V. Every intermediate goes through memory: this is the path the
 * flash kernels are timed against, not a fast path.
 * Arguments, layouts, cache types and errors as fa_prefill (any Sq, including decode shapes),
 * plus the caller-owned workspace:
 *   workspace   >= fa_standard_workspace_bytes(..., 1) bytes (one (b, KV head) unit at a time),
 *               256-byte aligned, need not be initialised. With more (up to
 *               fa_standard_workspace_bytes(..., 0), every unit at once) more units run per
 *               pass. Per unit it holds Sq * Hq/Hkv rows of S (f32) and P (16-bit) over the
 *               keys rounded up to 128, plus f16 copies of a q4_0 K or V (B * Sk * Hkv * D * 2
 *               bytes each). Calls sharing a workspace must be ordered on one stream.
 * fa_standard_workspace_bytes returns 0 for invalid sizes or an empty call.
 */
size_t fa_standard_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv_dtype,
                                   int units_per_pass);
int fa_standard_attention(const void *q, const void *k, const void *v, void *o,
                          int B, int Hq, int Hkv, int Sq, int Sk, int D,
                          int causal, int64_t causal_offset, float scale, int kv_dtype,
                          void *workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * Counter instances, for tests of the deferred rescale (mlxcel PR #2306, "What changed" and
 * "Test plan": O and l are rescaled only for a block whose maximum passes the row's frame by
 * more than the margin, which a chunked prefill on ordinary inputs hardly ever meets after its
 * first block; inputs whose scores climb along the keys are what make the branch run). They
 * run the same kernel source as fa_prefill / fa_decode with two counters per query row added,
 * and give the same output.
 *   counts   device int32 [B, Sq, Hq, 2], 8-byte aligned. Per query row (b, i, h):
 *            counts[..., 0] = how many times the row's softmax frame moved (the rescale test
 *            fired for the row; the first frame, taken from -inf, counts as one);
 *            counts[..., 1] = fa_prefill_stats: in how many 64-key tiles the row's wave ran
 *            the O rescale (it runs when any row of its 32-row block moved);
 *                             fa_decode_stats: how many key splits held keys for the row.
 *            fa_prefill_stats writes every row of the call; fa_decode_stats adds to the
 *            counters (every split of the row adds its own), so they must be zero first.
 * fa_prefill_stats: D = 128 and kv_dtype FA_KV_F16, FA_KV_BF16 or FA_KV_Q4_0, else
 * FA_ERR_UNSUPPORTED. fa_decode_stats: a q4_0 cache with at most 4 query rows per KV head
 * (Sq * Hq / Hkv <= 4) and Hkv a multiple of 4 (the head-group decode kernel), else
 * FA_ERR_UNSUPPORTED. Other arguments and errors as fa_prefill / fa_decode.
 */
int fa_prefill_stats(const void *q, const void *k, const void *v, void *o,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     int causal, int64_t causal_offset, float scale, int kv_dtype,
                     int32_t *counts, fa_stream_t stream);
int fa_decode_stats(const void *q, const void *k, const void *v, void *o,
                    int B, int Hq, int Hkv, int Sq, int Sk, int D,
                    int causal, int64_t causal_offset, float scale, int kv_dtype,
                    void *workspace, size_t workspace_bytes, int32_t *counts,
                    fa_stream_t stream);

/*
 * Dequantize n_blocks q4_0 blocks (18 bytes each, 2-byte aligned) with the same device
 * routine the attention kernels use. out_f32 receives the exact values (c - 8) * d as
 * float (n_blocks * 32 floats); out_f16 receives their f16 forms, rounded to nearest even
 * (n_blocks * 32 halves). Either output may be NULL, not both.
 */
int fa_dequant_q4_0(const void *blocks, int64_t n_blocks, float *out_f32, void *out_f16,
                    fa_stream_t stream);

/* Source element types of fa_quantize_q4_0. */
enum fa_src_dtype {
    FA_SRC_F32 = 0,
    FA_SRC_F16 = 1,
    FA_SRC_BF16 = 2,
};

/*
 * q4_0 cache writer, the step before the attention path: a new chunk's K and V rows are
 * quantized into the q4_0 cache the kernels read (the q4_0 KV cache of mi210-llm-stack,
 * "FlashAttention on gfx90a", "-ctk q4_0 -ctv q4_0"). Per 32 consecutive elements:
 * d = max|x| / 8 rounded to the nearest f16 (ties to even); element code
 * c = clamp(round_half_away(x / d) + 8, 0, 15) with x / d the correctly rounded f32 quotient
 * (so +max|x| gives 16, clamped to 15); every code is 8 when d = 0. The block is d (2 bytes,
 * little endian) then 16 bytes, byte t = c[t] | c[t + 16] << 4.
 *   x         device pointer to x_dtype elements: n_seq sequences of rows_per_seq rows of D
 *             elements (D > 0, a multiple of 32); sequence s starts at element
 *             s * x_seq_stride and its rows are contiguous. 16-byte aligned, and
 *             x_seq_stride * element size a multiple of 16.
 *   blocks    device pointer: sequence s's rows start at byte s * blocks_seq_stride and are
 *             contiguous, D / 32 * 18 bytes each. 2-byte aligned, blocks_seq_stride even.
 *             An append of S_new positions at pos to a [B, Smax, Hkv, D/32] q4_0 cache is
 *             blocks = cache + pos * Hkv * row bytes, n_seq = B, rows_per_seq = S_new * Hkv,
 *             blocks_seq_stride = Smax * Hkv * row bytes.
 * With n_seq > 1 each stride must cover a sequence (x_seq_stride >= rows_per_seq * D,
 * blocks_seq_stride >= rows_per_seq * D / 32 * 18). Elements must be finite, with max|x| / 8
 * inside the f16 range. Asynchronous on stream; the caller owns both buffers.
 * Returns FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_DTYPE, FA_ERR_ALIGN, FA_ERR_UNSUPPORTED
 * (more blocks than one launch takes) or FA_ERR_HIP.
 */
int fa_quantize_q4_0(const void *x, int x_dtype, void *blocks, int64_t n_seq,
                     int64_t rows_per_seq, int D, int64_t x_seq_stride,
                     int64_t blocks_seq_stride, fa_stream_t stream);

/*
 * Measurement export: a plain streaming read of `bytes` bytes (a multiple of 16) at buf
 * (16-byte aligned), the HBM read rate the memory-bound decode is compared with. Every thread
 * folds what it reads into one word; that word is written to *sink only if it equals magic,
 * so a sink is needed but normally never written. workgroups: grid size (0: 2048).
 */
int fa_measure_read(const void *buf, int64_t bytes, uint32_t *sink, uint32_t magic,
                    int workgroups, fa_stream_t stream);

/* Static text for a status code. */
const char *fa_strerror(int code);

/* Library version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
