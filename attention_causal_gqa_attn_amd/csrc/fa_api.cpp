// C ABI of libfa.so (declared in include/fa.h): argument validation, then one kernel launch
// (prefill) or two (decode: split + merge) on the caller's stream. Every check runs before
// the first HIP call, so a rejected call has launched nothing; the library allocates nothing.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "fa_device.h"
#include "fa_kernels.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr int64_t kMaxWorkgroups = (int64_t)UINT32_MAX / 256;   // 256-thread workgroups

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// a * b * c * d without int64 overflow (all >= 0); -1 on overflow.
int64_t mul4(int64_t a, int64_t b, int64_t c, int64_t d)
{
    const int64_t lim = INT64_MAX / 4;
    int64_t r = a;
    for (int64_t x : {b, c, d}) {
        if (x != 0 && r > lim / x)
            return -1;
        r *= x;
    }
    return r;
}

// Shared checks of fa_prefill / fa_decode. Fills `a` on success.
int check_attention(const void *q, const void *k, const void *v, void *o, int B, int Hq, int Hkv,
                    int Sq, int Sk, int D, int causal, int64_t offset, float scale, int kv_dtype,
                    fa::AttnArgs &a)
{
    if (kv_dtype != FA_KV_F16 && kv_dtype != FA_KV_BF16 && kv_dtype != FA_KV_Q4_0 &&
        kv_dtype != FA_KV_F16_Q4_0 && kv_dtype != FA_KV_Q4_0_F16)
        return FA_ERR_DTYPE;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0)
        return FA_ERR_SHAPE;
    if (D != 64 && D != 128)
        return FA_ERR_UNSUPPORTED;
    if (!(std::isfinite(scale) && scale > 0.0f))
        return FA_ERR_VALUE;
    const int64_t nq = mul4(B, Sq, Hq, D);
    const int64_t nk = mul4(B, Sk, Hkv, D);
    if (nq < 0 || nk < 0 || Sk > INT32_MAX - 2 * 64)
        return FA_ERR_SHAPE;
    // per-thread tile offsets are 32-bit: 64 key rows of all KV heads must span < 4 GiB
    if ((int64_t)Hkv * D * 2 * 64 > (int64_t)UINT32_MAX)
        return FA_ERR_UNSUPPORTED;
    if ((nq > 0 && (!q || !o)) || (nk > 0 && (!k || !v)))
        return FA_ERR_NULL;
    // q4_0 blocks need 4-byte alignment, 16-bit caches 16
    const uintptr_t k_align = fa::kv_k(kv_dtype) == fa::KV_Q4_0 ? 4 : 16;
    const uintptr_t v_align = fa::kv_v(kv_dtype) == fa::KV_Q4_0 ? 4 : 16;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, k_align) || !aligned(v, v_align))
        return FA_ERR_ALIGN;

    // offsets beyond these bounds change nothing: every key visible, or none
    if (offset > (int64_t)Sk)
        offset = Sk;
    if (offset < -(int64_t)Sq - 1)
        offset = -(int64_t)Sq - 1;

    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Sk = Sk;
    a.D = D;
    a.G = Hq / Hkv;
    a.kv = kv_dtype;
    a.causal = causal ? 1 : 0;
    a.offset = offset;
    a.c = scale * 1.4426950408889634f;
    return FA_OK;
}

int64_t visible_end(int Sq, int Sk, int causal, int64_t offset)
{
    if (!causal)
        return Sk;
    int64_t e = (int64_t)Sq - 1 + offset + 1;
    if (e > Sk)
        e = Sk;
    return e < 0 ? 0 : e;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// ---- fixed scratch of fa_decode_noalloc -------------------------------------------------------
// The decode workspace of fa_decode_noalloc lives in this file-scope device array, one copy per
// GPU, held until the process ends. Host code never uses the array's name as an address (on
// the host it is only a stand-in for the symbol): each device's copy is looked up once with
// hipGetSymbolAddress, with that device current, and the pointer is kept per device.
constexpr size_t kNoAllocScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`; FA_ERR_HIP if it cannot be found.
int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return FA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_prefill(const void *q, const void *k, const void *v, void *o, int B, int Hq, int Hkv,
               int Sq, int Sk, int D, int causal, int64_t causal_offset, float scale,
               int kv_dtype, fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    if (fa::prefill_grid(a).n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_prefill(a, (hipStream_t)stream));
}

size_t fa_prefill_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                                  int64_t causal_offset, int kv_dtype)
{
    fa::AttnArgs a;
    // sizes only: any non-null, aligned stand-in pointers pass the checks
    const void *nz = (const void *)(uintptr_t)4096;
    if (check_attention(nz, nz, nz, (void *)nz, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                        1.0f, kv_dtype, a) != FA_OK)
        return 0;
    return fa::prefill_split_plan(a).workspace_bytes;
}

int fa_prefill_split(const void *q, const void *k, const void *v, void *o, int B, int Hq,
                     int Hkv, int Sq, int Sk, int D, int causal, int64_t causal_offset,
                     float scale, int kv_dtype, void *workspace, size_t workspace_bytes,
                     fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    const fa::PrefillSplit sp = fa::prefill_split_plan(a);
    if (fa::prefill_grid(a).n_wg + sp.n_tail > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    if (sp.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < sp.workspace_bytes)
            return FA_ERR_WORKSPACE;
        if (!aligned(workspace, 16))
            return FA_ERR_ALIGN;
    }
    return hip_status(fa::launch_prefill_split(a, sp, workspace, (hipStream_t)stream));
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk < 0 || Hq % Hkv != 0 ||
        (D != 64 && D != 128))
        return 0;
    // the largest split count any causal offset can produce for these sizes, over the
    // kernels the cache types select
    size_t bytes = 0;
    for (int kv : {FA_KV_F16, FA_KV_Q4_0}) {
        const size_t nb =
            fa::decode_grid(B, Hq, Hkv, Sq, Sk, D, /*kend=*/Sk, /*bound=*/true, kv).workspace_bytes;
        bytes = nb > bytes ? nb : bytes;
    }
    return bytes;
}

int fa_decode(const void *q, const void *k, const void *v, void *o, int B, int Hq, int Hkv,
              int Sq, int Sk, int D, int causal, int64_t causal_offset, float scale, int kv_dtype,
              void *workspace, size_t workspace_bytes, fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if ((int64_t)(Hq / Hkv) * Sq > 16)
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    const fa::DecodeGrid g = fa::decode_grid(B, Hq, Hkv, Sq, Sk, D,
                                             visible_end(Sq, Sk, a.causal, a.offset), false,
                                             a.kv);
    if (g.n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    if (g.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < g.workspace_bytes)
            return FA_ERR_WORKSPACE;
        if (!aligned(workspace, 16))
            return FA_ERR_ALIGN;
    }
    return hip_status(fa::launch_decode(a, g, workspace, (hipStream_t)stream));
}

int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o, int B, int Hq,
                      int Hkv, int Sq, int Sk, int D, int causal, int64_t causal_offset,
                      float scale, int kv_dtype, fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if ((int64_t)(Hq / Hkv) * Sq > 16)
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    const fa::DecodeGrid g = fa::decode_grid(B, Hq, Hkv, Sq, Sk, D,
                                             visible_end(Sq, Sk, a.causal, a.offset), false,
                                             a.kv);
    if (g.n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    if (g.workspace_bytes > kNoAllocScratchBytes)
        return FA_ERR_TOO_LARGE;
    // every partial row the merge reads is written by the split kernel of the same call, so
    // nothing in the scratch has to start at zero
    void *ws = nullptr;
    const int sc = scratch_of_current_device(&ws);
    if (sc != FA_OK)
        return sc;
    return hip_status(fa::launch_decode(a, g, ws, (hipStream_t)stream));
}

int fa_prefill_stats(const void *q, const void *k, const void *v, void *o, int B, int Hq,
                     int Hkv, int Sq, int Sk, int D, int causal, int64_t causal_offset,
                     float scale, int kv_dtype, int32_t *counts, fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if (D != 128 || (kv_dtype != FA_KV_F16 && kv_dtype != FA_KV_BF16 && kv_dtype != FA_KV_Q4_0))
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    if (!counts)
        return FA_ERR_NULL;
    if (!aligned(counts, 8))
        return FA_ERR_ALIGN;
    if (fa::prefill_grid(a).n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_prefill(a, (hipStream_t)stream, nullptr, nullptr, counts));
}

int fa_decode_stats(const void *q, const void *k, const void *v, void *o, int B, int Hq,
                    int Hkv, int Sq, int Sk, int D, int causal, int64_t causal_offset,
                    float scale, int kv_dtype, void *workspace, size_t workspace_bytes,
                    int32_t *counts, fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if ((int64_t)(Hq / Hkv) * Sq > 16)
        return FA_ERR_UNSUPPORTED;
    if (!fa::q4_grouped(kv_dtype, (Hq / Hkv) * Sq, Hkv))
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    if (!counts)
        return FA_ERR_NULL;
    if (!aligned(counts, 8))
        return FA_ERR_ALIGN;
    const fa::DecodeGrid g = fa::decode_grid(B, Hq, Hkv, Sq, Sk, D,
                                             visible_end(Sq, Sk, a.causal, a.offset), false,
                                             a.kv);
    if (g.n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    if (g.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < g.workspace_bytes)
            return FA_ERR_WORKSPACE;
        if (!aligned(workspace, 16))
            return FA_ERR_ALIGN;
    }
    return hip_status(fa::launch_decode(a, g, workspace, (hipStream_t)stream, nullptr, counts));
}

size_t fa_standard_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv_dtype,
                                   int units_per_pass)
{
    fa::AttnArgs a;
    const void *nz = (const void *)(uintptr_t)4096;
    if (check_attention(nz, nz, nz, (void *)nz, B, Hq, Hkv, Sq, Sk, D, 0, 0, 1.0f, kv_dtype,
                        a) != FA_OK || (int64_t)B * Sq == 0)
        return 0;
    return fa::standard_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv_dtype, units_per_pass);
}

int fa_standard_attention(const void *q, const void *k, const void *v, void *o, int B, int Hq,
                          int Hkv, int Sq, int Sk, int D, int causal, int64_t causal_offset,
                          float scale, int kv_dtype, void *workspace, size_t workspace_bytes,
                          fa_stream_t stream)
{
    fa::AttnArgs a;
    const int rc = check_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    if (fa::standard_max_workgroups(B, Hq, Hkv, Sq, Sk, D, kv_dtype) > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    const size_t need = fa::standard_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv_dtype, 1);
    if (!workspace || workspace_bytes < need)
        return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return FA_ERR_ALIGN;
    return hip_status(fa::launch_standard(a, scale, workspace, workspace_bytes,
                                          (hipStream_t)stream));
}

int fa_dequant_q4_0(const void *blocks, int64_t n_blocks, float *out_f32, void *out_f16,
                    fa_stream_t stream)
{
    if (n_blocks < 0 || n_blocks > INT64_MAX / 64)
        return FA_ERR_SHAPE;
    if (n_blocks == 0)
        return FA_OK;
    if (!blocks || (!out_f32 && !out_f16))
        return FA_ERR_NULL;
    if (!aligned(blocks, 2) || !aligned(out_f32, 4) || !aligned(out_f16, 4))
        return FA_ERR_ALIGN;
    if ((n_blocks + 255) / 256 > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_dequant_q4_0(blocks, n_blocks, out_f32, out_f16,
                                              (hipStream_t)stream));
}

int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, void *o,
                    const int32_t *block_table, const int32_t *seq_lens, int B, int Hq,
                    int Hkv, int Sq, int D, int max_pages, int n_pages, int causal, float scale,
                    int kv_dtype, void *workspace, size_t workspace_bytes, fa_stream_t stream)
{
    if (max_pages < 0 || n_pages < 0 || max_pages > (INT32_MAX - 2 * 64) / 64)
        return FA_ERR_SHAPE;
    const int Sk = max_pages * 64;                  // keys a block-table row can address
    fa::AttnArgs a;
    // the causal offset is per sequence (its queries are its last Sq positions)
    const int rc = check_attention(q, k_pages, v_pages, o, B, Hq, Hkv, Sq, Sk, D, causal, 0,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if (mul4(n_pages, 64, Hkv, D) < 0)
        return FA_ERR_SHAPE;
    if ((int64_t)(Hq / Hkv) * Sq > 16)
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    if (max_pages > 0 && n_pages == 0)
        return FA_ERR_SHAPE;
    if (!block_table || !seq_lens)
        return FA_ERR_NULL;
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
        return FA_ERR_ALIGN;
    const fa::DecodeGrid g = fa::decode_grid(B, Hq, Hkv, Sq, Sk, D, Sk, false, a.kv);
    if (g.n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    if (g.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < g.workspace_bytes)
            return FA_ERR_WORKSPACE;
        if (!aligned(workspace, 16))
            return FA_ERR_ALIGN;
    }
    const fa::PagedKV pk{block_table, seq_lens, max_pages, n_pages};
    return hip_status(fa::launch_decode(a, g, workspace, (hipStream_t)stream, &pk));
}

int fa_prefill_paged(const void *q, const void *k_pages, const void *v_pages, void *o,
                     const int32_t *block_table, const int32_t *seq_lens, const int32_t *q_lens,
                     int B, int Hq, int Hkv, int Sq, int D, int max_pages, int n_pages,
                     int causal, float scale, int kv_dtype, fa_stream_t stream)
{
    if (max_pages < 0 || n_pages < 0 || max_pages > (INT32_MAX - 2 * 64) / 64)
        return FA_ERR_SHAPE;
    const int Sk = max_pages * 64;                  // keys a block-table row can address
    fa::AttnArgs a;
    // the causal offset is per sequence (its queries are its last q_lens[b] positions)
    const int rc = check_attention(q, k_pages, v_pages, o, B, Hq, Hkv, Sq, Sk, D, causal, 0,
                                   scale, kv_dtype, a);
    if (rc != FA_OK)
        return rc;
    if (mul4(n_pages, 64, Hkv, D) < 0)
        return FA_ERR_SHAPE;
    if (max_pages > fa::kPrefillMaxPages)
        return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Sq == 0)
        return FA_OK;
    if (max_pages > 0 && n_pages == 0)
        return FA_ERR_SHAPE;
    if (!block_table || !seq_lens)
        return FA_ERR_NULL;
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(q_lens, 4))
        return FA_ERR_ALIGN;
    if (fa::prefill_grid(a).n_wg > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    const fa::PagedKV pk{block_table, seq_lens, max_pages, n_pages};
    return hip_status(fa::launch_prefill(a, (hipStream_t)stream, &pk, q_lens));
}

int fa_quantize_q4_0(const void *x, int x_dtype, void *blocks, int64_t n_seq,
                     int64_t rows_per_seq, int D, int64_t x_seq_stride,
                     int64_t blocks_seq_stride, fa_stream_t stream)
{
    if (x_dtype != FA_SRC_F32 && x_dtype != FA_SRC_F16 && x_dtype != FA_SRC_BF16)
        return FA_ERR_DTYPE;
    if (n_seq < 0 || rows_per_seq < 0 || D <= 0 || D % 32)
        return FA_ERR_SHAPE;
    if (rows_per_seq > INT64_MAX / D)
        return FA_ERR_SHAPE;
    const int64_t elems = rows_per_seq * D;             // per sequence
    const int64_t per = elems / 32;                     // blocks per sequence
    if (n_seq == 0 || per == 0)
        return FA_OK;
    if (per > INT64_MAX / n_seq || elems > INT64_MAX / 18)
        return FA_ERR_SHAPE;
    if (n_seq > 1 && (x_seq_stride < elems || blocks_seq_stride < per * 18 ||
                      x_seq_stride > INT64_MAX / 4 / n_seq ||
                      blocks_seq_stride > INT64_MAX / n_seq))
        return FA_ERR_SHAPE;
    if (!x || !blocks)
        return FA_ERR_NULL;
    const int64_t esz = x_dtype == FA_SRC_F32 ? 4 : 2;
    if (!aligned(x, 16) || (n_seq > 1 && (x_seq_stride * esz) % 16) || !aligned(blocks, 2) ||
        (n_seq > 1 && blocks_seq_stride % 2))
        return FA_ERR_ALIGN;
    if ((n_seq * per + 255) / 256 > kMaxWorkgroups)
        return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_quantize_q4_0(x, x_dtype, blocks, n_seq, per, x_seq_stride,
                                               blocks_seq_stride, (hipStream_t)stream));
}

int fa_measure_read(const void *buf, int64_t bytes, uint32_t *sink, uint32_t magic,
                    int workgroups, fa_stream_t stream)
{
    if (bytes < 0 || bytes % 16 || workgroups < 0 || workgroups > (1 << 20))
        return FA_ERR_SHAPE;
    if (bytes == 0)
        return FA_OK;
    if (!buf || !sink)
        return FA_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return FA_ERR_ALIGN;
    return hip_status(fa::launch_read(buf, bytes / 16, sink, magic,
                                      workgroups > 0 ? workgroups : 2048, (hipStream_t)stream));
}

const char *fa_strerror(int code)
{
    switch (code) {
    case FA_OK:
        return "ok";
    case FA_ERR_NULL:
        return "a required pointer is NULL";
    case FA_ERR_SHAPE:
        return "invalid sizes (negative, Hq not a multiple of Hkv, or too large)";
    case FA_ERR_DTYPE:
        return "unknown kv_dtype";
    case FA_ERR_UNSUPPORTED:
        return "unsupported combination (head dim not 64 or 128, decode rows > 16, grid too large)";
    case FA_ERR_WORKSPACE:
        return "decode workspace missing or too small";
    case FA_ERR_ALIGN:
        return "misaligned pointer (16 bytes; q4_0 K/V 4 bytes)";
    case FA_ERR_HIP:
        return "HIP runtime error at launch";
    case FA_ERR_VALUE:
        return "scale must be finite and positive";
    case FA_ERR_TOO_LARGE:
        return "fa_decode_noalloc: the call needs more than the fixed scratch "
               "(FA_NOALLOC_SCRATCH_BYTES); use fa_decode with a workspace";
    default:
        return "unknown status code";
    }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
