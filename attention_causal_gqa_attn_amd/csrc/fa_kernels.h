// Internal interface between the C ABI (fa_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a prefill or decode launch needs; filled and validated by the C ABI layer.
struct AttnArgs {
    const void *q, *k, *v;
    void *o;
    int B, Hq, Hkv, Sq, Sk, D;
    int G;              // query heads per KV head
    int kv;             // KV_F16, KV_BF16 or KV_Q4_0
    int causal;
    int64_t offset;     // query i sits at absolute position i + offset
    float c;            // scale * log2(e)
};

// Prefill workgroup decomposition (fa_prefill16.hip): `waves` (4) waves of 64 query rows; hpw
// heads of one KV group by qsub 64-row sub-blocks (hpw * qsub = waves); heads beyond `waves`
// of a group go to further chunks.
struct PrefillGrid {
    int waves, hpw, qsub, n_qblk, n_hchunk;
    int64_t n_wg;
};
PrefillGrid prefill_grid(const AttnArgs &a);
struct PagedKV;
// paged: a paged cache (a.Sk = max_pages * 64, a.offset unused); q_lens (paged only, may be
// null): sequence b's query count, rows [0, q_lens[b]) of its Sq; stats (contiguous caches,
// D = 128, one cache type for K and V; else hipErrorInvalidValue): the counter instance, two
// int32 per query row [B, Sq, Hq, 2]
hipError_t launch_prefill(const AttnArgs &a, hipStream_t stream, const PagedKV *paged = nullptr,
                          const int32_t *q_lens = nullptr, int32_t *stats = nullptr);
PrefillGrid prefill16_grid(const AttnArgs &a);
hipError_t launch_prefill16(const AttnArgs &a, const PrefillGrid &g, hipStream_t stream,
                            const PagedKV *paged = nullptr, const int32_t *q_lens = nullptr,
                            int32_t *stats = nullptr);
// the paged prefill keeps a sequence's page numbers in LDS: at most this many per sequence
constexpr int kPrefillMaxPages = 4096;
// Balanced causal prefill (fa_prefill_split, contiguous caches; a q4_0 tensor at D = 128
// only): units holding more than `cap` tiles leave their tiles past the cap to the workgroup of their mirror query block
// (n - 1 - q), which runs them after its own unit; the two parts are merged through a caller
// workspace: kSplitCounterBytes of arrival counters (zero between calls), then the parts'
// partial rows. n_main: workgroups (one per unit); n_tail: split units, 0 when nothing splits
// (plain prefill).
constexpr size_t kSplitCounterBytes = 4096;
// parts > 0: the key split for shapes with few units (each unit's tiles cut into `parts` runs,
// one workgroup each, n_main = units x parts; a merge kernel follows); 0: the pairing above.
struct PrefillSplit {
    int q_split, cap;
    int64_t n_main, n_tail;
    size_t workspace_bytes;
    int parts;
    // q4_0 tensors widened to f16 in the workspace first (bit 0: K, bit 1: V), each copy
    // deq_bytes long, the first at deq_off; the split then runs on the 16-bit copies
    int deq;
    size_t deq_off, deq_bytes;
};
PrefillSplit prefill_split_plan(const AttnArgs &a);
hipError_t launch_prefill_split(const AttnArgs &a, const PrefillSplit &sp, void *workspace,
                                hipStream_t stream);

// Decode: n_split key ranges per (b, KV head); rows = G * Sq query rows per KV head (<= 16).
struct DecodeGrid {
    int rows, n_split, split_len;   // split_len: keys per split, a multiple of 64
    int64_t n_wg;
    size_t workspace_bytes;
};
// kend: keys any row can see, [0, kend). With bound = true the result's workspace_bytes is
// the largest any kend <= Sk can need (the split count is not monotone in kend). kv picks the
// kernel, which sets how many workgroups share a key range.
DecodeGrid decode_grid(int B, int Hq, int Hkv, int Sq, int Sk, int D, int64_t kend, bool bound,
                       int kv);
bool q4_grouped(int kv, int rows, int Hkv);
// Paged K/V (fa_decode_paged): pages of 64 keys ([n_pages][64][Hkv][row]); sequence b's key j
// is in page block_table[b * max_pages + j / 64]; seq_lens[b] keys (device arrays).
struct PagedKV {
    const int32_t *block_table, *seq_lens;
    int max_pages, n_pages;
};
// stats (q4_0 caches taking the head-group kernel only, else hipErrorInvalidValue): the
// counter instance, two int32 per query row [B, Sq, Hq, 2] that every split adds to
hipError_t launch_decode(const AttnArgs &a, const DecodeGrid &g, void *workspace,
                         hipStream_t stream, const PagedKV *paged = nullptr,
                         int32_t *stats = nullptr);

// Standard (non-flash) attention, the comparison arm (fa_standard.hip): workspace bytes for
// units_per_pass (b, KV head) units at a time (<= 0: all of them), the largest grid it
// launches, and the launch (a.k / a.v as fa_prefill; the workspace holds at least one unit).
size_t standard_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv,
                                int units_per_pass);
int64_t standard_max_workgroups(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv);
hipError_t launch_standard(const AttnArgs &a, float scale, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

// Streaming read of n16 16-byte chunks with `grid` workgroups (fa_measure.hip).
hipError_t launch_read(const void *buf, int64_t n16, uint32_t *sink, uint32_t magic, int grid,
                       hipStream_t stream);

hipError_t launch_dequant_q4_0(const void *blocks, int64_t n_blocks, float *out_f32,
                               void *out_f16, hipStream_t stream);
// src: 0 f32, 1 f16, 2 bf16 (fa_src_dtype)
hipError_t launch_quantize_q4_0(const void *x, int src, void *blocks, int64_t n_seq,
                                int64_t blocks_per_seq, int64_t x_seq_stride,
                                int64_t blk_seq_stride, hipStream_t stream);

}  // namespace fa
