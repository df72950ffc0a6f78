// Decode kernels: split-K attention for few query rows per KV head, then a log-sum-exp merge.
//
// The rows of one KV head (its G query heads times Sq query tokens, at most 16) share every
// K/V element, so a workgroup streams one range of keys ("split") of one (b, KV head) through
// LDS once and computes all rows against it. Many splits run at once to keep HBM busy; each
// writes its partial softmax state (frame f, sum l, unnormalised output row) and a second
// kernel combines the splits of a row:
//     F = max_s f_s,   L = sum_s l_s 2^(f_s - F),   O = sum_s O_s 2^(f_s - F) / L
// (log2 units). A q4_0 cache is dequantized on the way into LDS by the same tile loader as
// the prefill kernel.
//
// Inside a workgroup the 4 waves take 16 keys each of every 64-key tile:
//   S^T[16 keys][16 rows] = v_mfma_f32_16x16x32 (K from LDS, Q^T in registers);
//   the C layout puts 4 consecutive keys of one row in a lane, which is exactly the B operand
//   of v_mfma_f32_16x16x16 for O^T[16 d][16 rows] += V^T[16 d][16 keys] P^T;
//   each wave keeps its own deferred softmax frame per row (rescale only past the margin),
//   and the 4 waves' states are combined through LDS at the end of the split.
#include "fa_kernels.h"
#include "fa_tiles.h"

namespace fa {

// q4_0 decode with at most 4 query rows per KV head and a KV head count divisible by 4 takes
// the head-group kernel (one workgroup per 4 heads and key range)
bool q4_grouped(int kv, int rows, int Hkv) { return kv == KV_Q4_0 && rows <= 4 && Hkv % 4 == 0; }

namespace {

struct DecodeParams {
    AttnArgs a;
    int rows, n_split, split_len;
    int64_t kend;          // keys any row can see: [0, kend) (contiguous caches)
    float *part;           // [B][Hkv][n_split][rows][D + 2]
    // paged caches (block_table != nullptr): K and V are n_pages pages of kBN keys, each
    // [kBN][Hkv][row]; key j of sequence b is key j % kBN of page block_table[b * max_pages +
    // j / kBN]; sequence b has seq_lens[b] keys and its Sq queries are its last Sq positions
    const int32_t *block_table, *seq_lens;
    int max_pages, n_pages;
    // counter instance of the head-group q4_0 kernel: per query row (b, i, h) two int32 that
    // every split adds to (they must start at zero): the times the row's softmax frame moved
    // in the split (the deferred-rescale test fired, counting the split's first frame), and 1
    // for each split that held keys
    int32_t *stats;
};

// One sequence's keys: how many it has, how many its rows can see ([0, kend)), and the
// absolute position of its query 0.
struct SeqView {
    int64_t Sk, kend, offset;
};
__device__ __forceinline__ SeqView seq_view(const DecodeParams &p, int b)
{
    const AttnArgs &a = p.a;
    if (!p.block_table)
        return SeqView{a.Sk, p.kend, a.offset};
    const int64_t sk = min(max((int64_t)p.seq_lens[b], (int64_t)0), (int64_t)p.max_pages * kBN);
    return SeqView{sk, sk, sk - a.Sq};
}
// Byte offset of (b, key 0, KV head kvh) in K or V: contiguous caches are [B, Sk, Hkv, row];
// pages are shared by every sequence.
__device__ __forceinline__ int64_t head_off(const DecodeParams &p, int b, int kvh, int rowb)
{
    const AttnArgs &a = p.a;
    return p.block_table ? (int64_t)kvh * rowb : ((int64_t)b * a.Sk * a.Hkv + kvh) * rowb;
}
// Byte offset from the head's key-0 row to the 64-key tile at key k0 (a multiple of kBN); rows
// inside a tile are grow bytes apart in both layouts. A page index outside the page array is
// clamped into it: the result is then wrong, but every load stays inside the buffers.
// Paged: the offsets come from a run of up to 64 block-table entries held one per lane,
// fetched with one vector load when a tile falls outside it (at the first tile, then at most
// once per 64 table entries); a tile's page is taken with v_readlane, so no memory access
// sits between a tile's transfers. (A scalar load per tile would either wait in front of the
// transfers or, left in flight, turn every LDS wait of the compute into a wait for it, since
// scalar loads complete out of order.)
struct PageRun {
    int base = -(1 << 30);  // table index held by lane 0 (wave-uniform); none held yet
    int v = 0;              // lane l: entry base + l
    // fetch the run at tile k0 ahead of time (at kernel start, beside the sequence-length read,
    // so the two latencies overlap instead of adding up)
    __device__ __forceinline__ void prime(const DecodeParams &p, int b, int64_t k0, int lane)
    {
        if (p.block_table && p.max_pages > 0) {
            base = (int)min(k0 / kBN, (int64_t)p.max_pages - 1);
            v = p.block_table[(int64_t)b * p.max_pages + min(base + lane, p.max_pages - 1)];
        }
    }
    __device__ __forceinline__ int64_t off(const DecodeParams &p, int b, int64_t k0,
                                           uint32_t grow, int lane)
    {
        if (!p.block_table)
            return k0 * grow;
        const int j = (int)min(k0 / kBN, (int64_t)p.max_pages - 1);
        if (j < base || j >= base + 64) {
            base = j;
            v = p.block_table[(int64_t)b * p.max_pages + min(j + lane, p.max_pages - 1)];
        }
        int pg = __builtin_amdgcn_readlane(v, j - base);
        pg = min(max(pg, 0), p.n_pages - 1);
        return (int64_t)pg * kBN * grow;
    }
};

// One 64-key tile of the split: each wave takes 16 keys.
template <int D, bool BF>
__device__ __forceinline__ void decode_tile(const uint16_t *lk, const uint16_t *lv, int k0,
                                            int wave, int quad, int r, int64_t rowlim, float c,
                                            const u32x4 *qf, f32x4 *acc, float &frame,
                                            float &lsum)
{
    using Geo = TileGeom<D>;
    const int kw = k0 + 16 * wave;                  // this wave's first key
    if (!__any(kw <= rowlim))                       // wave-uniform: no row sees these keys
        return;
    f32x4 sc = (f32x4){};
    const uint16_t *kr = lk + (16 * wave + r) * Geo::kStride + 8 * quad;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        sc = mfma16<BF>(*(const u32x4 *)(kr + 32 * kk), qf[kk], sc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (kw + 4 * quad + i > rowlim)
            sc[i] = -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = pair_max(mx);
    const float m2 = mx * c;
    const bool need = m2 > frame + kRescaleMarginLog2;
    if (__any(need)) {
        const float alpha = need ? exp2_fast(frame - m2) : 1.0f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            acc[dt] *= alpha;
        lsum *= alpha;
        frame = need ? m2 : frame;
    }
    const float fr = (frame == -INFINITY) ? 0.0f : frame;
    u32x2 pf;
    {
        const float p0 = exp2_fast(__builtin_fmaf(sc[0], c, -fr));
        const float p1 = exp2_fast(__builtin_fmaf(sc[1], c, -fr));
        const float p2 = exp2_fast(__builtin_fmaf(sc[2], c, -fr));
        const float p3 = exp2_fast(__builtin_fmaf(sc[3], c, -fr));
        pf[0] = pack2<BF>(p0, p1);
        pf[1] = pack2<BF>(p2, p3);
        lsum = sum2<BF>(pf[1], sum2<BF>(pf[0], lsum));
    }
    const uint16_t *vr = lv + r * Geo::vStride + 16 * wave + 4 * quad;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = mfma16k16<BF>(*(const u32x2 *)(vr + 16 * dt * Geo::vStride), pf, acc[dt]);
}

// Combine per-wave softmax states held in LDS and write the split's partial [O, F, L] rows.
// Wave w's row rr: unnormalised output at o0[w * ows + rr * D + d], frame f0[w * fws + rr],
// sum l0[w * fws + rr]. A wave that saw no key has frame -inf and contributes nothing.
template <int D>
__device__ __forceinline__ void write_partial(const DecodeParams &p, const float *o0, int ows,
                                              const float *f0, const float *l0, int fws,
                                              int b, int kvh, int s, int t)
{
    const AttnArgs &a = p.a;
    float *out = p.part + (((int64_t)b * a.Hkv + kvh) * p.n_split + s) * p.rows * (D + 2);
    for (int e = t; e < p.rows * D; e += kThreads) {
        const int rr = e / D, d = e % D;
        float F = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            F = fmaxf(F, f0[w * fws + rr]);
        float o = 0.0f, l = 0.0f;
        if (F != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sw = exp2_fast(f0[w * fws + rr] - F);   // 0 for an empty wave
                o += sw * o0[w * ows + rr * D + d];
                l += sw * l0[w * fws + rr];
            }
        }
        out[rr * (D + 2) + d] = o;
        if (d == 0) {
            out[rr * (D + 2) + D] = F;
            out[rr * (D + 2) + D + 1] = l;
        }
    }
}

// Combine the 4 waves' softmax states of each row (through LDS at cmb, 4*16*(D+2) floats)
// and write the split's partial [F, L, O] rows.
template <int D>
__device__ __forceinline__ void decode_combine(const DecodeParams &p, float *cmb, int b, int kvh,
                                               int s, int t, int wave, int quad, int r,
                                               const f32x4 *acc, float frame, float lsum)
{
    lsum += __shfl_xor(lsum, 16, 64);
    lsum = pair_sum(lsum);
    float *cmb_o = cmb;                             // [4 waves][16 rows][D]
    float *cmb_f = cmb_o + 4 * 16 * D;              // [4][16]
    float *cmb_l = cmb_f + 64;                      // [4][16]
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cmb_o[(wave * 16 + r) * D + 16 * dt + 4 * quad + i] = acc[dt][i];
    if (quad == 0) {
        cmb_f[wave * 16 + r] = frame;
        cmb_l[wave * 16 + r] = lsum;
    }
    __syncthreads();
    write_partial<D>(p, cmb_o, 16 * D, cmb_f, cmb_l, 16, b, kvh, s, t);
}

// Tiles whose global loads are in flight at once per workgroup: decode has little work per
// byte, so keeping HBM busy needs several tiles outstanding. The q4_0 staging registers are
// small (10 per thread per tile), the 16-bit ones are not.
template <int KV>
constexpr int kDecodeSets = KV == KV_Q4_0 ? 2 : 1;

// Waves per SIMD the register budget is sized for: 4 workgroups per CU for q4_0 (small
// staging registers), 3 for the 16-bit caches (16 staging registers per thread).
template <int KV>
constexpr int kDecodeOccupancy = KV == KV_Q4_0 ? 4 : 3;

template <int D, int KV>
__global__ __launch_bounds__(kThreads, kDecodeOccupancy<KV>) void decode_split_kernel(DecodeParams p)
{
    constexpr bool BF = (KV == KV_BF16);
    constexpr int NSETS = kDecodeSets<KV>;
    using Geo = TileGeom<D>;
    // one K + V^T tile, reused afterwards for the cross-wave combine
    constexpr int kLdsElems = Geo::stage > 4 * 16 * D * 2 + 256 ? Geo::stage
                                                                : 4 * 16 * D * 2 + 256;
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];

    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int quad = lane >> 4, r = lane & 15;     // C layout: keys 4*quad + i, row r

    // KV head fastest: the Hkv workgroups of one key range go to one XCD together, and since
    // a key's rows of all KV heads are contiguous they share that XCD's L2 lines
    int rest = xcd_remap(blockIdx.x, gridDim.x);
    const int kvh = rest % a.Hkv;
    rest /= a.Hkv;
    const int s = rest % p.n_split;
    const int b = rest / p.n_split;
    PageRun pr;
    pr.prime(p, b, (int64_t)s * p.split_len, lane);
    const SeqView sv = seq_view(p, b);

    const int64_t ks = (int64_t)s * p.split_len;
    const int64_t ke = min(ks + p.split_len, sv.kend);
    const int nb = ke > ks ? (int)((ke - ks + kBN - 1) / kBN) : 0;

    // row r = qi * G + hl; rows >= p.rows are padding
    const bool row_on = r < p.rows;
    const int qi = row_on ? r / a.G : 0;
    const int hl = row_on ? r % a.G : 0;
    const int h = kvh * a.G + hl;
    int64_t rowlim = ke - 1;                        // last key this row may see in the split
    if (a.causal)
        rowlim = min(rowlim, (int64_t)qi + sv.offset);
    if (!row_on)
        rowlim = -1;

    // Q^T as B operands: lane holds row r, d = 32*kk + 8*quad .. +7
    u32x4 qf[D / 32];
    {
        const uint16_t *qp = (const uint16_t *)a.q + (((int64_t)b * a.Sq + qi) * a.Hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qf[kk] = row_on ? *(const u32x4 *)(qp + 32 * kk + 8 * quad) : (u32x4){};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            settle(qf[kk]);
    }

    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = (f32x4){};
    float frame = -INFINITY, lsum = 0.0f;

    // tile kb is staged by loader kb % NSETS; NSETS tiles are in flight ahead of the compute
    TileLoader<D, KV> ld[NSETS];
#pragma unroll
    for (int u = 0; u < NSETS; ++u)
        ld[u].init(a.k, a.v, head_off(p, b, kvh, 1), a.Hkv, (int)sv.Sk, t);
    // bytes between consecutive keys of K and of V (they differ for mixed caches)
    const uint32_t growk = (uint32_t)a.Hkv * kv_row_bytes(kv_k(KV), D);
    const uint32_t growv = (uint32_t)a.Hkv * kv_row_bytes(kv_v(KV), D);
    auto load_set = [&](int u, int k0) {
        ld[u].load(k0, pr.off(p, b, k0, growk, lane), pr.off(p, b, k0, growv, lane));
    };
    uint16_t *lk = lds, *lv = lds + Geo::kElems;
    int kb0 = 0;
    if (nb >= 2 * NSETS) {
        // Steady state: the prologue and every iteration issue the same loads in the same
        // order, so the compiler's in-order load accounting stays exact and storing set u
        // waits only for set u, not for the sets issued after it.
#pragma unroll
        for (int u = 0; u < NSETS; ++u)
            load_set(u, (int)ks + u * kBN);
        for (; kb0 + 2 * NSETS <= nb; kb0 += NSETS) {
#pragma unroll
            for (int u = 0; u < NSETS; ++u) {
                ld[u].store(lk, lv);
                __syncthreads();
                load_set(u, (int)ks + (kb0 + u + NSETS) * kBN);
                decode_tile<D, BF>(lk, lv, (int)ks + (kb0 + u) * kBN, wave, quad, r, rowlim,
                                   a.c, qf, acc, frame, lsum);
                __syncthreads();
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < NSETS; ++u)
            if (u < nb)
                load_set(u, (int)ks + u * kBN);
    }
    // tail: the last tiles (their loads are already in flight), loading only what exists
    for (; kb0 < nb; kb0 += NSETS) {
#pragma unroll
        for (int u = 0; u < NSETS; ++u) {
            const int kb = kb0 + u;
            if (kb < nb) {                          // uniform over the workgroup
                ld[u].store(lk, lv);
                __syncthreads();
                if (kb + NSETS < nb)
                    load_set(u, (int)ks + (kb + NSETS) * kBN);
                decode_tile<D, BF>(lk, lv, (int)ks + kb * kBN, wave, quad, r, rowlim, a.c, qf,
                                   acc, frame, lsum);
                __syncthreads();
            }
        }
    }

    decode_combine<D>(p, (float *)lds, b, kvh, s, t, wave, quad, r, acc, frame, lsum);
}

// ---- q4_0 caches: raw blocks through an LDS-DMA ring -----------------------------------------
// A key's q4_0 row of one KV head (D/32 blocks of 18 bytes) is cut into 12-byte chunks, each
// copied into a 16-byte LDS slot by global_load_lds_dwordx3, in the slot layout the tile
// loader reads (padding slots get a repeat of the row's last chunk); a whole tile (64 keys of
// K, then of V) is NI wave-wide transfers, NIW per wave. Tiles run two ahead through kRS = 3
// raw stages; the tile loader dequantizes a raw stage into the f16 K / V^T tiles as before.
constexpr int kRS = 3;

// One 12-byte LDS-DMA transfer per lane: gbase + voff -> LDS lds_base + 16 * lane. Issued from
// asm for the same reason as in the prefill kernel (the compiler would wait for every
// outstanding transfer before each LDS read); the kernel orders the LDS data with explicit
// vmcnt waits and barriers, and nothing else in it uses M0. An SALU write of M0 needs one wait
// state before the LDS-DMA load that reads it.
__device__ __forceinline__ void dma12(const uint8_t *gbase, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds_base) : "memory");
}

// s_waitcnt immediate: at most `vm` vector-memory ops outstanding, all LDS ops done
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_q4_kernel(DecodeParams p)
{
    using Geo = TileGeom<D>;
    using LD = TileLoader<D, KV_Q4_0>;
    constexpr int CPR = LD::RAW_CPR;                // 12-byte chunks per key row
    constexpr int ST = LD::RAW_STRIDE;              // slots per row (CPR rounded up to odd)
    constexpr int RAW_T = 16 * LD::RAW_SLOTS;       // bytes of one tensor's raw tile in LDS
    constexpr int NI = 2 * ST;                      // wave-wide transfers per tile (K, then V)
    constexpr int NIW = (NI + 3) / 4;               // per wave (surplus ones repeat the last)
    constexpr int kLdsElems = Geo::stage > 4 * 16 * (D + 2) * 2 ? Geo::stage
                                                                 : 4 * 16 * (D + 2) * 2;
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
    __shared__ __attribute__((aligned(16))) uint8_t raw[kRS * 2 * RAW_T];

    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int quad = lane >> 4, r = lane & 15;

    int rest = xcd_remap(blockIdx.x, gridDim.x);
    const int kvh = rest % a.Hkv;
    rest /= a.Hkv;
    const int s = rest % p.n_split;
    const int b = rest / p.n_split;
    PageRun pr;
    pr.prime(p, b, (int64_t)s * p.split_len, lane);
    const SeqView sv = seq_view(p, b);

    const int64_t ks = (int64_t)s * p.split_len;
    const int64_t ke = min(ks + p.split_len, sv.kend);
    const int nb = ke > ks ? (int)((ke - ks + kBN - 1) / kBN) : 0;

    const bool row_on = r < p.rows;
    const int qi = row_on ? r / a.G : 0;
    const int hl = row_on ? r % a.G : 0;
    const int h = kvh * a.G + hl;
    int64_t rowlim = ke - 1;
    if (a.causal)
        rowlim = min(rowlim, (int64_t)qi + sv.offset);
    if (!row_on)
        rowlim = -1;

    u32x4 qf[D / 32];
    {
        const uint16_t *qp = (const uint16_t *)a.q + (((int64_t)b * a.Sq + qi) * a.Hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qf[kk] = row_on ? *(const u32x4 *)(qp + 32 * kk + 8 * quad) : (u32x4){};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            settle(qf[kk]);
    }
    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = (f32x4){};
    float frame = -INFINITY, lsum = 0.0f;

    // ---- transfers: this wave's m-th transfer of a tile is i = min(wave + 4 m, NI - 1) -----
    const uint32_t grow = (uint32_t)a.Hkv * LD::ROWB;            // bytes between keys
    const int64_t head0 = head_off(p, b, kvh, LD::ROWB);
    const uint8_t *kg = (const uint8_t *)a.k + head0, *vg = (const uint8_t *)a.v + head0;
    const uint32_t raw0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)raw;
    uint32_t crow[NIW], ccol[NIW];
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
        const int i = min(wave + 4 * m, NI - 1);
        const int sl = (i % ST) * 64 + lane;        // slot within the tensor's tile
        const int rr = sl / (32 * ST), kp = (sl % (32 * ST)) / ST, j = sl % ST;
        crow[m] = (uint32_t)(2 * kp + rr);
        ccol[m] = (uint32_t)(12 * min(j, CPR - 1));
    }
    auto dma_tile = [&](int kb) {
        const int k0 = (int)ks + kb * kBN;
        const uint32_t last = (uint32_t)min((int64_t)kBN - 1, sv.Sk - 1 - k0);
        const uint32_t stage = raw0 + (uint32_t)((kb % kRS) * 2 * RAW_T);
        const int64_t toff = pr.off(p, b, k0, grow, lane);
#pragma unroll
        for (int m = 0; m < NIW; ++m) {
            const int i = min(wave + 4 * m, NI - 1);
            const bool is_v = i >= ST;
            const uint8_t *gt = (is_v ? vg : kg) + toff;
            const uint32_t lbase = stage + (uint32_t)((is_v ? RAW_T : 0) + (i % ST) * 64 * 16);
            dma12(gt, min(crow[m], last) * grow + ccol[m],
                  __builtin_amdgcn_readfirstlane(lbase));
        }
    };
    // before the barrier of tile kb its raw stage is complete; tile kb+1 may be in flight
    auto wait_raw = [&](bool next_pending) {
        if (next_pending)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(NIW));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        asm volatile("s_barrier" ::: "memory");
    };

    LD ld;                                          // its raw-stage reads and f16 stores only
    ld.init(a.k, a.v, 0, a.Hkv, (int)sv.Sk, t);
    uint16_t *lk = lds, *lv = lds + Geo::kElems;
    if (nb > 0)
        dma_tile(0);
    if (nb > 1)
        dma_tile(1);
    for (int kb = 0; kb < nb; ++kb) {
        // raw(kb) resident; every wave is done with the f16 tiles of kb-1 and (dequantized in
        // iteration kb-1) the raw stage that tile kb+2 now goes into
        wait_raw(kb + 1 < nb);
        if (kb + 2 < nb)
            dma_tile(kb + 2);
        const uint8_t *rs = raw + (kb % kRS) * 2 * RAW_T;
        ld.load_raw(rs, rs + RAW_T);
        ld.store(lk, lv);
        __syncthreads();
        decode_tile<D, false>(lk, lv, (int)ks + kb * kBN, wave, quad, r, rowlim, a.c, qf, acc,
                              frame, lsum);
    }
    __syncthreads();
    decode_combine<D>(p, (float *)lds, b, kvh, s, t, wave, quad, r, acc, frame, lsum);
}

// ---- q4_0 caches, at most 4 query rows per KV head --------------------------------------------
// v_mfma_f32_4x4x4_16b_f16 computes 16 independent 4x4 products with K = 4: lane i + 4*blk
// holds row i of block blk's A (its 4 k values), column i of its B, and column i of its D
// (register r = row r). The 4 columns are the query rows of a KV head, so no score, exp or
// output element is padding. One wave carries one KV head's attention over whole tiles.
//
// The codes are never dequantized element by element. An f16 bit pattern with only low
// mantissa bits set is the subnormal n * 2^-24, exact, and the MFMA multiplies subnormal f16
// inputs exactly, so a code byte masked in place with 0x0F is its low nibble n * 2^-24 and
// masked with 0xF0 its high nibble times 16 * 2^-24. The block scale d and the offset 8 are
// applied outside the per-element path:
//   scores:  s = sum_b D_b * (2^-24 sum_{e in b} n_e q_e - 2^-21 sum_{e in b} q_e), D_b = 2^24 d_b
//            (one accumulator per block b, started at the q term; high nibbles meet q / 16);
//   output:  o_e = sum_k P_k d_b(k) (n_ke - 8) = 2^24 sum_k P'_k n_ke 2^-24 - 8 sum_k P'_k with
//            P'_k = P_k d_b(k) (f16) as the B operand and the sum of P' kept beside O.
constexpr int kQ4Rows = 4;

__device__ __forceinline__ f32x4 mfma4(uint32_t a0, uint32_t a1, u32x2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, (u32x2){a0, a1}),
                                              __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// x of lane (l & ~3) + I: DPP quad broadcast
template <int I>
__device__ __forceinline__ float quad_bcast(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              I * 0x55, 0xF, 0xF, false));
}
// max over lanes {l, l ^ 4, l ^ 8, l ^ 12} (one 16-lane row, same l % 4): DPP row rotates
__device__ __forceinline__ float row4_max(float x)
{
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                    0x124, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                    0x128, 0xF, 0xF, false)));
    return x;
}
// max over the 16-lane row pair {row, row ^ 1}: v_permlane16_swap on two copies (as in
// lane_halves for the 32-lane halves)
__device__ __forceinline__ float rowpair_max(float x)
{
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return fmaxf(a, b);
}

// max / sum over the 64 lanes of a wave, the result in every lane: DPP row rotates inside the
// 16-lane rows, then v_permlane16_swap and v_permlane32_swap across them (no LDS round trips)
__device__ __forceinline__ float wave_max(float x)
{
    x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                   0x121, 0xF, 0xF, false)));
    x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                   0x122, 0xF, 0xF, false)));
    x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                   0x124, 0xF, 0xF, false)));
    x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                   0x128, 0xF, 0xF, false)));
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return pair_max(vmax(a, b));
}
__device__ __forceinline__ float wave_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121,
                                                            0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122,
                                                            0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124,
                                                            0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128,
                                                            0xF, 0xF, false));
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return pair_sum(a + b);
}

// Wait until at most N vector-memory operations of this wave are outstanding; also a compiler
// memory fence, so no LDS read of the landed data moves above it.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// One wave's attention of the <= 4 query rows of one KV head over q4_0 tiles in LDS whose key
// rows (the head's D/32 blocks of 18 bytes) are RS bytes apart.
template <int D, int RS>
struct Q4Head {
    static constexpr int NB = D / 32;               // q4_0 blocks per key row
    static constexpr int ROWB = 18 * NB;            // bytes of the head's key row
    static constexpr int ROWDW = ROWB / 4;
    static constexpr int KGC = 16 / NB;             // 4-key groups per P.V chunk
    static constexpr int NCH = kBN / (4 * KGC);     // P.V chunks per tile

    int lane, j, bq, kg;
    int64_t rowlim, lim0;
    uint32_t vlo, vhi, vsh, vsc;
    int psrc;
    u32x2 qlo[NB][4], qhi[NB][4];
    f32x4 sinit[NB];
    f32x4 oacc[8];                                  // P.V, MFMA q + 4 hh: byte q, nibble hh
    float frame, lsum, csum;
    int nmove;                                      // frame moves (the counter instance)

    // Query rows j = lane % 4 (qi * G + hl; rows >= p.rows are padding, computed and never
    // written) of KV head kvh of batch b, over keys below ke.
    __device__ __forceinline__ void init(const DecodeParams &p, int b, int kvh, int64_t ke,
                                         int64_t offset, int lane_)
    {
        const AttnArgs &a = p.a;
        lane = lane_;
        j = lane & 3;
        const bool row_on = j < p.rows;
        const int qi = row_on ? j / a.G : 0;
        const int hl = row_on ? j % a.G : 0;
        const int h = kvh * a.G + hl;
        rowlim = ke - 1;
        if (a.causal)
            rowlim = min(rowlim, (int64_t)qi + offset);
        if (!row_on)
            rowlim = -1;
        lim0 = ke - 1;                              // smallest limit of a real row (row 0)
        if (a.causal)
            lim0 = min(lim0, offset);

        // B operands of the score MFMAs: row j of q in the k order of the A operands. Code
        // dword pp of block bb holds bytes 4 pp .. 4 pp + 3; masked as in scores() its slots
        // are elements 32 bb + 4 pp + {0, 2, 1, 3} (low nibbles) and 16 more (high nibbles).
        const uint16_t *qp = (const uint16_t *)a.q + (((int64_t)b * a.Sq + qi) * a.Hq + h) * D;
        u32x4 qv[NB][4];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                qv[bb][u] = row_on ? *(const u32x4 *)(qp + 32 * bb + 8 * u) : (u32x4){};
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                settle(qv[bb][u]);
        const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            float qs = 0.0f;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                // element pairs (e, e + 1): the low half of the block in qv[bb][0..1], the
                // high half in qv[bb][2..3]
                const uint32_t l0 = qv[bb][pp / 2][2 * (pp % 2)];
                const uint32_t l1 = qv[bb][pp / 2][2 * (pp % 2) + 1];
                const uint32_t h0 = qv[bb][2 + pp / 2][2 * (pp % 2)];
                const uint32_t h1 = qv[bb][2 + pp / 2][2 * (pp % 2) + 1];
                qlo[bb][pp] = (u32x2){perm(l1, l0, 0x05040100u), perm(l1, l0, 0x07060302u)};
                const uint32_t x0 = perm(h1, h0, 0x05040100u), x1 = perm(h1, h0, 0x07060302u);
                qhi[bb][pp] = (u32x2){
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x0) * sixteenth),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x1) * sixteenth)};
                const f32x2 a0 = unpack2<false>(l0), a1 = unpack2<false>(l1);
                const f32x2 c0 = unpack2<false>(h0), c1 = unpack2<false>(h1);
                qs += (a0[0] + a0[1]) + (a1[0] + a1[1]) + (c0[0] + c0[1]) + (c1[0] + c1[1]);
            }
            const float q8 = -0x1p-21f * qs;
            sinit[bb] = (f32x4){q8, q8, q8, q8};
        }

        // P.V roles: A row pp = lane % 4 (code dword pp of block bq of the 4 keys of group kg),
        // B / D column j = lane % 4, block bq * KGC + kg = lane / 4. Even blocks start 2 bytes
        // into a dword: their code dword is spliced from two.
        bq = (lane >> 2) / KGC;
        kg = (lane >> 2) % KGC;
        const int pp = lane & 3;
        vlo = (uint32_t)(RS * 4 * kg + 18 * bq + 4 * pp + ((bq & 1) ? 2 : 0));
        vhi = vlo + ((bq & 1) ? 0u : 4u);
        vsh = (bq & 1) ? 0u : 16u;
        vsc = (uint32_t)(RS * 4 * kg + 18 * bq);                // scale of block bq
        psrc = (lane & (4 * KGC - 1)) * 4;                       // + 16 KGC c for chunk c

#pragma unroll
        for (int m = 0; m < 8; ++m)
            oacc[m] = (f32x4){};
        frame = -INFINITY;
        lsum = 0.0f;
        csum = 0.0f;
        nmove = 0;
    }

    // Scores of the tile's 64 keys (from key k0; kt = the head's key row 0 in LDS) and the
    // softmax state update; returns P as two packed f16 pairs (keys 4 blk + 0..3 of row j).
    // Lane l supplies key l's K row as A; D lane j + 4 blk, register r is key 4 blk + r.
    template <bool STATS = false>
    __device__ __forceinline__ u32x2 scores(const uint8_t *kt, int64_t k0, float c)
    {
        uint32_t w[ROWDW];
        const uint8_t *kr = kt + RS * lane;
        if constexpr (ROWB % 8 == 0) {
#pragma unroll
            for (int u = 0; u < ROWDW / 2; ++u) {
                const u32x2 x = *(const u32x2 *)(kr + 8 * u);
                w[2 * u] = x[0];
                w[2 * u + 1] = x[1];
            }
        } else {
#pragma unroll
            for (int u = 0; u < ROWDW; ++u)
                w[u] = *(const uint32_t *)(kr + 4 * u);
        }
        // the NB accumulators' chains interleaved, so consecutive MFMAs are independent
        f32x4 sacc[NB];
        float dsc[NB];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t cw[NB], y[NB];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                if (bb % 2 == 0)
                    cw[bb] = __builtin_amdgcn_alignbit(w[9 * bb / 2 + q + 1], w[9 * bb / 2 + q], 16);
                else
                    cw[bb] = w[(18 * bb + 2) / 4 + q];
                y[bb] = cw[bb] >> 8;
            }
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
                sacc[bb] = mfma4(cw[bb] & 0x000F000Fu, y[bb] & 0x000F000Fu, qlo[bb][q],
                                 q == 0 ? sinit[bb] : sacc[bb]);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
                sacc[bb] = mfma4(cw[bb] & 0x00F000F0u, y[bb] & 0x00F000F0u, qhi[bb][q], sacc[bb]);
        }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            const uint32_t dbits = (bb % 2 == 0) ? (w[9 * bb / 2] & 0xFFFFu)
                                                 : (w[(18 * bb - 2) / 4] >> 16);
            dsc[bb] = (float)__builtin_bit_cast(_Float16, (uint16_t)dbits) * 0x1p24f;
        }
        float sc[4];
        {
            float d0[NB], d1[NB], d2[NB], d3[NB];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                d0[bb] = quad_bcast<0>(dsc[bb]);
                d1[bb] = quad_bcast<1>(dsc[bb]);
                d2[bb] = quad_bcast<2>(dsc[bb]);
                d3[bb] = quad_bcast<3>(dsc[bb]);
            }
            sc[0] = d0[0] * sacc[0][0];
            sc[1] = d1[0] * sacc[0][1];
            sc[2] = d2[0] * sacc[0][2];
            sc[3] = d3[0] * sacc[0][3];
#pragma unroll
            for (int bb = 1; bb < NB; ++bb) {
                sc[0] = __builtin_fmaf(d0[bb], sacc[bb][0], sc[0]);
                sc[1] = __builtin_fmaf(d1[bb], sacc[bb][1], sc[1]);
                sc[2] = __builtin_fmaf(d2[bb], sacc[bb][2], sc[2]);
                sc[3] = __builtin_fmaf(d3[bb], sacc[bb][3], sc[3]);
            }
        }
        if (k0 + kBN - 1 > lim0) {                  // wave-uniform: a row limit falls here
            const int64_t key = k0 + 4 * (lane >> 2);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (key + r > rowlim)
                    sc[r] = -INFINITY;
        }

        // softmax state of row j (deferred rescale)
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = row4_max(mx);
        mx = rowpair_max(mx);
        mx = pair_max(mx);
        const float m2 = mx * c;
        const bool need = m2 > frame + kRescaleMarginLog2;
        if constexpr (STATS)
            nmove += need ? 1 : 0;
        if (__any(need)) {
            const float alpha = need ? exp2_fast(frame - m2) : 1.0f;
#pragma unroll
            for (int m = 0; m < 8; ++m)
                oacc[m] *= alpha;
            lsum *= alpha;
            csum *= alpha;
            frame = need ? m2 : frame;
        }
        const float fr = (frame == -INFINITY) ? 0.0f : frame;
        const uint32_t pk0 = pack2<false>(exp2_fast(__builtin_fmaf(sc[0], c, -fr)),
                                          exp2_fast(__builtin_fmaf(sc[1], c, -fr)));
        const uint32_t pk1 = pack2<false>(exp2_fast(__builtin_fmaf(sc[2], c, -fr)),
                                          exp2_fast(__builtin_fmaf(sc[3], c, -fr)));
        lsum = sum2<false>(pk1, sum2<false>(pk0, lsum));
        return (u32x2){pk0, pk1};
    }

    // This lane's V operands of the tile (vt = the head's V row 0 in LDS), all read up front
    // so their LDS latency overlaps the scores: per chunk c and key k, the two dwords the code
    // dword is spliced from, and the block scale.
    uint32_t vlo_w[NCH][4], vhi_w[NCH][4];
    uint16_t vdq[NCH][4];
    __device__ __forceinline__ void load_v(const uint8_t *vt)
    {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint8_t *vr = vt + RS * 4 * KGC * c;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vlo_w[c][k] = *(const uint32_t *)(vr + RS * k + vlo);
                vhi_w[c][k] = *(const uint32_t *)(vr + RS * k + vhi);
                vdq[c][k] = *(const uint16_t *)(vr + RS * k + vsc);
            }
        }
    }

    // O += P V over the tile whose operands load_v() read.
    __device__ __forceinline__ void pv(u32x2 pk)
    {
        uint32_t pb0[NCH], pb1[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            // P of keys 4 (KGC c + kg) + 0..3, row j, from the score lane j + 4 kg + 16 KGC c
            const int src = psrc + 16 * KGC * c;
            pb0[c] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)pk[0]);
            pb1[c] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)pk[1]);
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t b0 = pb0[c], b1 = pb1[c];
            uint32_t cw[4];
            uint16_t dq[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                cw[k] = __builtin_amdgcn_alignbit(vhi_w[c][k], vlo_w[c][k], vsh);
                dq[k] = vdq[c][k];
            }
            const f16x2 s01 = __builtin_bit_cast(f16x2, (uint32_t)dq[0] | ((uint32_t)dq[1] << 16));
            const f16x2 s23 = __builtin_bit_cast(f16x2, (uint32_t)dq[2] | ((uint32_t)dq[3] << 16));
            const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, b0) * s01);
            const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, b1) * s23);
            csum = sum2<false>(p23, sum2<false>(p01, csum));
            const u32x2 pb = {p01, p23};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t sel = 0x0C000C00u | ((4u + q) << 16) | (uint32_t)q;
                const uint32_t u01 = perm(cw[1], cw[0], sel), u23 = perm(cw[3], cw[2], sel);
                oacc[q] = mfma4(u01 & 0x000F000Fu, u23 & 0x000F000Fu, pb, oacc[q]);
                oacc[q + 4] = mfma4(u01 & 0x00F000F0u, u23 & 0x00F000F0u, pb, oacc[q + 4]);
            }
        }
    }

    // Reduce over the key-group lanes. Afterwards lanes with kg == 0 hold the unnormalised
    // output of row j for block bq: o(r, q, hh) is element 32 bq + 4 r + q + 16 hh; every lane
    // holds row j's frame and sum.
    __device__ __forceinline__ void reduce()
    {
#pragma unroll
        for (int sh = 4; sh < 4 * KGC; sh *= 2) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    oacc[m][r] += __shfl_xor(oacc[m][r], sh, 64);
            csum += __shfl_xor(csum, sh, 64);
        }
#pragma unroll
        for (int sh = 4; sh < 64; sh *= 2)
            lsum += __shfl_xor(lsum, sh, 64);
    }
    __device__ __forceinline__ float out(int r, int q, int hh) const
    {
        return (hh ? 0x1p20f : 0x1p24f) * oacc[q + 4 * hh][r] - 8.0f * csum;
    }
};

// One dword LDS-DMA transfer per lane: gbase + voff -> LDS lds_base + 4 * lane.
__device__ __forceinline__ void dma4(const uint8_t *gbase, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds_base) : "memory");
}
// One 16-byte LDS-DMA transfer per lane: gbase + voff -> LDS lds_base + 16 * lane.
__device__ __forceinline__ void dma16x(const uint8_t *gbase, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds_base) : "memory");
}

// (a) Head groups: a workgroup takes 4 adjacent KV heads (one per wave) over one key range. A
// key's rows of the 4 heads are contiguous in memory (4 * 18 D/32 bytes, a multiple of 16), so
// the waves together move whole 16-byte chunks with LDS-DMA: tile rows of S 16-byte slots (S
// odd, the last a repeat when the data is an even number of chunks), so the 16-byte K row
// reads of 16 consecutive keys fall into distinct LDS banks. NSTG stages; one barrier a tile.
template <int D>
struct Q4G {
    static constexpr int NH = 4;                    // KV heads per workgroup, one per wave
    static constexpr int ROWB = 18 * (D / 32);
    static constexpr int GB = NH * ROWB;            // bytes of the group's key row
    static constexpr int DS = GB / 16;              // its 16-byte chunks
    static constexpr int S = DS | 1;                // LDS slots per key row
    static constexpr int RS = 16 * S;
    static constexpr int TB = kBN * RS;             // one tensor's tile in LDS
    static constexpr int NI = 2 * S;                // wave-wide transfers per tile (K, then V)
    static constexpr int NIW = (NI + 3) / 4;        // per wave (surplus ones repeat the last)
    static constexpr int STAGE = 2 * TB;
    static constexpr int NSTG = 2;                  // stages (tiles in flight + 1)
    static constexpr int OCC = 2;                   // workgroups per CU (LDS-bound)
    static_assert(GB % 16 == 0, "group rows are whole 16-byte chunks");
};
constexpr int kQ4gWorkgroups = 256 * Q4G<128>::OCC;

template <int D, bool STATS = false>
__global__ __launch_bounds__(kThreads, Q4G<D>::OCC) void decode_q4g_kernel(DecodeParams p)
{
    using G = Q4G<D>;
    using H = Q4Head<D, G::RS>;
    constexpr int NSTG = G::NSTG, NIW = G::NIW, S = G::S;
    __shared__ __attribute__((aligned(16))) uint8_t lds[NSTG * G::STAGE];

    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

    // head group fastest: the groups of one key range go to one XCD together and share its
    // L2 lines (a key's rows of all KV heads are contiguous)
    const int ngrp = a.Hkv / G::NH;
    int rest = xcd_remap(blockIdx.x, gridDim.x);
    const int grp = rest % ngrp;
    rest /= ngrp;
    const int s = rest % p.n_split;
    const int b = rest / p.n_split;
    const int kvh = grp * G::NH + wave;
    PageRun pr;
    pr.prime(p, b, (int64_t)s * p.split_len, lane);
    const SeqView sv = seq_view(p, b);

    const int64_t ks = (int64_t)s * p.split_len;
    const int64_t ke = min(ks + p.split_len, sv.kend);
    const int nb = ke > ks ? (int)((ke - ks + kBN - 1) / kBN) : 0;

    H hd;
    hd.init(p, b, kvh, ke, sv.offset, lane);

    // transfers: this wave's m-th of a tile is i = min(wave + 4 m, NI - 1); i < S moves K slot
    // column i (slots 64 i .. 64 i + 63 of the tile), else V column i - S
    const uint32_t grow = (uint32_t)a.Hkv * G::ROWB;                    // bytes between keys
    const int64_t g0 = head_off(p, b, grp * G::NH, G::ROWB);
    const uint8_t *kgl = (const uint8_t *)a.k + g0, *vgl = (const uint8_t *)a.v + g0;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)lds);
    uint32_t crow[NIW], ccol[NIW];
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
        const int i = min(wave + 4 * m, G::NI - 1);
        const int sl = (i % S) * 64 + lane;
        crow[m] = (uint32_t)(sl / S);
        ccol[m] = 16u * (uint32_t)min(sl % S, G::DS - 1);
    }
    auto dma_tile = [&](int kb) {
        const int64_t k0 = ks + (int64_t)kb * kBN;
        const uint32_t last = (uint32_t)min((int64_t)kBN - 1, sv.Sk - 1 - k0);
        const uint32_t st = lds0 + (uint32_t)((kb % NSTG) * G::STAGE);
        const int64_t toff = pr.off(p, b, k0, grow, lane);
#pragma unroll
        for (int m = 0; m < NIW; ++m) {
            const int i = min(wave + 4 * m, G::NI - 1);
            const bool is_v = i >= S;
            dma16x((is_v ? vgl : kgl) + toff, min(crow[m], last) * grow + ccol[m],
                   __builtin_amdgcn_readfirstlane(st + (uint32_t)((is_v ? G::TB : 0) +
                                                                  (i % S) * 1024)));
        }
    };

#pragma unroll
    for (int u = 0; u < NSTG - 1; ++u)
        if (u < nb)
            dma_tile(u);
    for (int kb = 0; kb < nb; ++kb) {
        // tile kb landed for every wave; every wave is done with tile kb - 1, whose stage the
        // next transfer refills
        if constexpr (NSTG >= 4) {
            if (kb + 2 < nb)
                wait_vm<2 * NIW>();
            else if (kb + 1 < nb)
                wait_vm<NIW>();
            else
                wait_vm<0>();
        } else if constexpr (NSTG == 3) {
            if (kb + 1 < nb)
                wait_vm<NIW>();
            else
                wait_vm<0>();
        } else {
            wait_vm<0>();
        }
        asm volatile("s_barrier" ::: "memory");
        if (kb + NSTG - 1 < nb)
            dma_tile(kb + NSTG - 1);
        const uint8_t *kt = lds + (kb % NSTG) * G::STAGE + wave * G::ROWB;
        hd.load_v(kt + G::TB);
        const u32x2 pk = hd.template scores<STATS>(kt, ks + (int64_t)kb * kBN, a.c);
        hd.pv(pk);
    }

    if constexpr (STATS) {
        // one lane per row adds this split's counts
        if (lane < p.rows && nb > 0) {
            const int qi = lane / a.G, h = kvh * a.G + lane % a.G;
            int32_t *st = p.stats + 2 * (((int64_t)b * a.Sq + qi) * a.Hq + h);
            atomicAdd(st, hd.nmove);
            atomicAdd(st + 1, 1);
        }
    }
    // this wave's head: write the split's partial rows directly
    hd.reduce();
    if (hd.kg == 0 && hd.j < p.rows) {
        float *out = p.part + ((((int64_t)b * a.Hkv + kvh) * p.n_split + s) * p.rows + hd.j) *
                                  (D + 2);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    out[32 * hd.bq + 16 * hh + 4 * r + q] = hd.out(r, q, hh);
        if (hd.bq == 0) {
            out[D] = hd.frame;
            out[D + 1] = hd.lsum;
        }
    }
}

// (b) Any KV head count: each wave owns every 4th tile of the workgroup's key range of one
// head (kb = wave, wave + 4, ...) and two raw LDS stages of its own, filled by dword LDS-DMA
// (the tile's 64 K rows, then its 64 V rows, densely packed); nothing in the loop waits for
// another wave, and the 4 waves' states are combined through LDS at the end.
template <int D>
struct Q4W {
    static constexpr int ROWB = 18 * (D / 32);      // bytes per key row
    static constexpr int ROWDW = ROWB / 4;
    static constexpr int TILEB = kBN * ROWB;        // one tensor's raw tile
    static constexpr int NX = TILEB / 256;          // dword LDS-DMA transfers per tensor tile
    static constexpr int NV = NX < 9 ? NX : 9;      // distinct lane offsets among them
    static constexpr int RSTEP = 64 * NV / ROWDW;   // key rows spanned by NV transfers
    static constexpr int STAGE = 2 * TILEB;         // K rows then V rows
    static constexpr int WAVE_LDS = 2 * STAGE;      // two stages per wave
    static_assert((64 * NV) % ROWDW == 0, "offset reuse");
    static_assert(4 * D + 8 <= WAVE_LDS / 4, "combine scratch fits in a wave's stages");
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_q4w_kernel(DecodeParams p)
{
    using W = Q4W<D>;
    using H = Q4Head<D, W::ROWB>;
    constexpr int ROWDW = W::ROWDW, TILEB = W::TILEB, NX = W::NX, NV = W::NV;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * W::WAVE_LDS];

    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

    int rest = xcd_remap(blockIdx.x, gridDim.x);
    const int kvh = rest % a.Hkv;
    rest /= a.Hkv;
    const int s = rest % p.n_split;
    const int b = rest / p.n_split;
    PageRun pr;
    pr.prime(p, b, (int64_t)s * p.split_len, lane);
    const SeqView sv = seq_view(p, b);

    const int64_t ks = (int64_t)s * p.split_len;
    const int64_t ke = min(ks + p.split_len, sv.kend);
    const int nb = ke > ks ? (int)((ke - ks + kBN - 1) / kBN) : 0;
    const int ni = nb > wave ? (nb - wave + 3) / 4 : 0;      // tiles wave + 4 i, i < ni

    H hd;
    hd.init(p, b, kvh, ke, sv.offset, lane);

    // transfers: lane offsets of the first NV dword transfers of a tensor tile
    const uint32_t grow = (uint32_t)a.Hkv * W::ROWB;                    // bytes between keys
    const int64_t head0 = head_off(p, b, kvh, W::ROWB);
    const uint8_t *kgl = (const uint8_t *)a.k + head0, *vgl = (const uint8_t *)a.v + head0;
    uint8_t *wl = lds + wave * W::WAVE_LDS;
    const uint32_t wl0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)wl);
    uint32_t vo[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) {
        const int e = 64 * m + lane;
        vo[m] = (uint32_t)(e / ROWDW) * grow + 4u * (uint32_t)(e % ROWDW);
    }
    auto dma_tile = [&](int i) {
        const int64_t k0 = ks + (int64_t)(wave + 4 * i) * kBN;
        const uint32_t st = wl0 + (uint32_t)((i & 1) * W::STAGE);
        const int64_t last = min((int64_t)kBN - 1, sv.Sk - 1 - k0);
        const int64_t toff = pr.off(p, b, k0, grow, lane);
        if (last == kBN - 1) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int x = 0; x < NX; ++x)
                    dma4((tt ? vgl : kgl) + toff + (int64_t)(x / NV) * W::RSTEP * grow,
                         vo[x % NV], st + (uint32_t)(tt * TILEB + 256 * x));
        } else {
            // the sequence's last, partial tile: rows past its last key re-read that key (a
            // rolled loop, so the compiler cannot merge it into the common path with selects)
#pragma unroll 1
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll 1
                for (int x = 0; x < NX; ++x) {
                    const int e = 64 * x + lane;
                    const uint32_t row = (uint32_t)min(e / ROWDW, (int)last);
                    dma4((tt ? vgl : kgl) + toff, row * grow + 4u * (uint32_t)(e % ROWDW),
                         st + (uint32_t)(tt * TILEB + 256 * x));
                }
        }
    };

    if (ni > 0)
        dma_tile(0);
    if (ni > 1)
        dma_tile(1);
    for (int i = 0; i < ni; ++i) {
        const bool more = i + 1 < ni;
        const uint8_t *sk = wl + (i & 1) * W::STAGE;
        // tile i has landed (tile i + 1 may still be in flight)
        if (more)
            wait_vm<2 * NX>();
        else
            wait_vm<0>();
        hd.load_v(sk + TILEB);
        const u32x2 pk = hd.scores(sk, ks + (int64_t)(wave + 4 * i) * kBN, a.c);
        hd.pv(pk);
        if (i + 2 < ni)
            dma_tile(i + 2);
    }

    // this wave's state -> LDS (its own stage area; all its transfers have landed)
    hd.reduce();
    float *fo = (float *)wl;                        // [4 rows][D], then f[4], l[4]
    if (hd.kg == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fo[hd.j * D + 32 * hd.bq + 16 * hh + 4 * r + q] = hd.out(r, q, hh);
        if (hd.bq == 0) {
            fo[4 * D + hd.j] = hd.frame;
            fo[4 * D + 4 + hd.j] = hd.lsum;
        }
    }
    __syncthreads();
    const float *f0 = (const float *)lds;
    write_partial<D>(p, f0, W::WAVE_LDS / 4, f0 + 4 * D, f0 + 4 * D + 4, W::WAVE_LDS / 4, b,
                     kvh, s, t);
}

// More than 64 splits: one wave per (b, KV head, row), log-sum-exp merge of the row's n_split
// partials in a loop.
template <int D, bool BF>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p)
{
    __shared__ float wts[1024];
    const AttnArgs &a = p.a;
    const int lane = threadIdx.x;
    int rest = blockIdx.x;
    const int rr = rest % p.rows;
    rest /= p.rows;
    const int kvh = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int stride = p.rows * (D + 2);
    const float *base = p.part + ((int64_t)b * a.Hkv + kvh) * p.n_split * stride + rr * (D + 2);
    const int qi = rr / a.G, hl = rr % a.G;
    uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi) * a.Hq + kvh * a.G + hl) * D;

    float F = -INFINITY;
    for (int s = lane; s < p.n_split; s += 64)
        F = vmax(F, base[(int64_t)s * stride + D]);
    F = wave_max(F);
    float L = 0.0f;
    for (int s = lane; s < p.n_split; s += 64) {
        const float w = F == -INFINITY ? 0.0f : exp2_fast(base[(int64_t)s * stride + D] - F);
        wts[s] = w;
        L += w * base[(int64_t)s * stride + D + 1];
    }
    L = wave_sum(L);
    __syncthreads();
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;

    // the splits' loads are issued 16 at a time, so their latencies overlap
    for (int d2 = lane; d2 < D / 2; d2 += 64) {
        float o0 = 0.0f, o1 = 0.0f;
        int s = 0;
        for (; s + 16 <= p.n_split; s += 16) {
            f32x2 x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                x[u] = *(const f32x2 *)(base + (int64_t)(s + u) * stride + 2 * d2);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                o0 += wts[s + u] * x[u][0];
                o1 += wts[s + u] * x[u][1];
            }
        }
        for (; s < p.n_split; ++s) {
            const f32x2 x = *(const f32x2 *)(base + (int64_t)s * stride + 2 * d2);
            o0 += wts[s] * x[0];
            o1 += wts[s] * x[1];
        }
        *(uint32_t *)(op + 2 * d2) = pack2<BF>(o0 * inv, o1 * inv);
    }
}

// At most 64 splits: four waves per (b, KV head, row). Every split's output row, frame and
// sum is loaded in one round (wave w holds splits w, w + 4, ..., 16 per lane, so a lane has
// 16 loads in flight instead of 64), the frames and sums first so that the weights are formed
// while the outputs are in flight; split u's weight is lane u's, read back with v_readlane;
// the four waves' partial rows meet in LDS.
template <int D, bool BF>
__global__ __launch_bounds__(256) void decode_merge4_kernel(DecodeParams p)
{
    constexpr int E = D / 64;
    __shared__ float part[3][D];
    const AttnArgs &a = p.a;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rest = blockIdx.x;
    const int rr = rest % p.rows;
    rest /= p.rows;
    const int kvh = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int stride = p.rows * (D + 2);
    const float *base = p.part + ((int64_t)b * a.Hkv + kvh) * p.n_split * stride + rr * (D + 2);
    const int ns = p.n_split;
    const bool on = lane < ns;
    const f32x2 fl = *(const f32x2 *)(base + (int64_t)min(lane, ns - 1) * stride + D);
    float x[16][E];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const float *src = base + (int64_t)min(wave + 4 * u, ns - 1) * stride + E * lane;
        if constexpr (E == 2) {
            const f32x2 v2 = *(const f32x2 *)src;
            x[u][0] = v2[0];
            x[u][1] = v2[1];
        } else {
            x[u][0] = *src;
        }
    }
    const float f = on ? fl[0] : -INFINITY;
    const float l = on ? fl[1] : 0.0f;
    const float F = wave_max(f);
    const float w = (F == -INFINITY || !on) ? 0.0f : exp2_fast(f - F);
    const float L = wave_sum(w * l);
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        o[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const float wu = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), wave + 4 * u));
#pragma unroll
        for (int e = 0; e < E; ++e)
            o[e] += wu * x[u][e];
    }
    if (wave > 0)
#pragma unroll
        for (int e = 0; e < E; ++e)
            part[wave - 1][E * lane + e] = o[e];
    __syncthreads();
    if (wave > 0)
        return;
#pragma unroll
    for (int e = 0; e < E; ++e)
        o[e] += part[0][E * lane + e] + part[1][E * lane + e] + part[2][E * lane + e];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int qi = rr / a.G, hl = rr % a.G;
    uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi) * a.Hq + kvh * a.G + hl) * D;
    if constexpr (E == 2)
        *(uint32_t *)(op + 2 * lane) = pack2<BF>(o[0] * inv, o[1] * inv);
    else
        op[lane] = (uint16_t)(pack2<BF>(o[0] * inv, 0.0f) & 0xFFFFu);
}

// 65 to 16 NW splits: NW waves per (b, KV head, row), wave w holding splits w, w + NW, ...
// (16 per lane), so every split's row is again loaded in one round. A wave combines its own
// splits against its own largest frame (lanes 0..15 hold their frames and sums); the waves'
// partial rows, frames and sums then meet in LDS and are combined the same way (log-sum-exp
// of the waves' states, the merge applied twice).
template <int D, bool BF, int NW>
__global__ __launch_bounds__(64 * NW) void decode_mergew_kernel(DecodeParams p)
{
    constexpr int E = D / 64;
    __shared__ float part[NW][D];
    __shared__ float wfl[NW][2];
    const AttnArgs &a = p.a;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rest = blockIdx.x;
    const int rr = rest % p.rows;
    rest /= p.rows;
    const int kvh = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int stride = p.rows * (D + 2);
    const float *base = p.part + ((int64_t)b * a.Hkv + kvh) * p.n_split * stride + rr * (D + 2);
    const int ns = p.n_split;
    const int su = wave + NW * min(lane, 15);        // lane u < 16: split wave + NW u
    const bool on = lane < 16 && su < ns;
    const f32x2 fl = *(const f32x2 *)(base + (int64_t)min(su, ns - 1) * stride + D);
    float x[16][E];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const float *src = base + (int64_t)min(wave + NW * u, ns - 1) * stride + E * lane;
        if constexpr (E == 2) {
            const f32x2 v2 = *(const f32x2 *)src;
            x[u][0] = v2[0];
            x[u][1] = v2[1];
        } else {
            x[u][0] = *src;
        }
    }
    const float f = on ? fl[0] : -INFINITY;
    const float Fw = wave_max(f);
    const float w = (Fw == -INFINITY || !on) ? 0.0f : exp2_fast(f - Fw);
    const float Lw = wave_sum(w * (on ? fl[1] : 0.0f));
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        o[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const float wu = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
        for (int e = 0; e < E; ++e)
            o[e] += wu * x[u][e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        part[wave][E * lane + e] = o[e];
    if (lane == 0) {
        wfl[wave][0] = Fw;
        wfl[wave][1] = Lw;
    }
    __syncthreads();
    if (wave > 0)
        return;
    float F = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v)
        F = fmaxf(F, wfl[v][0]);
    float L = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        o[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const float c = (F == -INFINITY || wfl[v][0] == -INFINITY) ? 0.0f
                                                                    : exp2_fast(wfl[v][0] - F);
        L += c * wfl[v][1];
#pragma unroll
        for (int e = 0; e < E; ++e)
            o[e] += c * part[v][E * lane + e];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int qi = rr / a.G, hl = rr % a.G;
    uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi) * a.Hq + kvh * a.G + hl) * D;
    if constexpr (E == 2)
        *(uint32_t *)(op + 2 * lane) = pack2<BF>(o[0] * inv, o[1] * inv);
    else
        op[lane] = (uint16_t)(pack2<BF>(o[0] * inv, 0.0f) & 0xFFFFu);
}

template <int D, int KV>
hipError_t launch(const DecodeParams &p, int64_t n_wg, hipStream_t stream)
{
    if (p.stats && !(KV == KV_Q4_0 && q4_grouped(p.a.kv, p.rows, p.a.Hkv)))
        return hipErrorInvalidValue;
    if constexpr (KV == KV_Q4_0) {
        if (p.stats)
            hipLaunchKernelGGL((decode_q4g_kernel<D, true>), dim3((unsigned)n_wg),
                               dim3(kThreads), 0, stream, p);
        else if (q4_grouped(p.a.kv, p.rows, p.a.Hkv))
            hipLaunchKernelGGL((decode_q4g_kernel<D>), dim3((unsigned)n_wg), dim3(kThreads), 0,
                               stream, p);
        else if (p.rows <= kQ4Rows)
            hipLaunchKernelGGL((decode_q4w_kernel<D>), dim3((unsigned)n_wg), dim3(kThreads), 0,
                               stream, p);
        else
            hipLaunchKernelGGL((decode_q4_kernel<D>), dim3((unsigned)n_wg), dim3(kThreads), 0,
                               stream, p);
    }
    else
        hipLaunchKernelGGL((decode_split_kernel<D, KV>), dim3((unsigned)n_wg), dim3(kThreads), 0,
                           stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t n_rows = (int64_t)p.a.B * p.a.Hkv * p.rows;
    if (p.n_split <= 64)
        hipLaunchKernelGGL((decode_merge4_kernel<D, KV == KV_BF16>), dim3((unsigned)n_rows),
                           dim3(256), 0, stream, p);
    else if (p.n_split <= 128)
        hipLaunchKernelGGL((decode_mergew_kernel<D, KV == KV_BF16, 8>), dim3((unsigned)n_rows),
                           dim3(512), 0, stream, p);
    else if (p.n_split <= 256)
        hipLaunchKernelGGL((decode_mergew_kernel<D, KV == KV_BF16, 16>), dim3((unsigned)n_rows),
                           dim3(1024), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_merge_kernel<D, KV == KV_BF16>), dim3((unsigned)n_rows),
                           dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// Split choice: about 512 workgroups in all (two per CU), each split a whole number of
// 64-key tiles and at least one tile.
constexpr int64_t kTargetWorkgroups = 512;

DecodeGrid decode_grid(int B, int Hq, int Hkv, int Sq, int Sk, int D, int64_t kend, bool bound,
                       int kv)
{
    DecodeGrid g;
    g.rows = (Hq / Hkv) * Sq;
    const int64_t heads = (int64_t)B * Hkv;
    // workgroups per key range: one per KV head, or one per group of 4 heads
    const bool grouped = q4_grouped(kv, g.rows, Hkv);
    const int64_t per = grouped ? heads / 4 : heads;
    const int64_t target = grouped ? kQ4gWorkgroups : kTargetWorkgroups;
    int64_t want = per > 0 ? (target + per - 1) / per : 1;
    if (want > 1024)
        want = 1024;     // the merge kernel keeps one weight per split in LDS
    const int64_t tiles = (kend + kBN - 1) / kBN;
    const int64_t tiles_per = tiles > 0 ? (tiles + want - 1) / want : 1;
    g.split_len = (int)(tiles_per * kBN);
    g.n_split = tiles > 0 ? (int)((tiles + tiles_per - 1) / tiles_per) : 1;
    if (bound) {
        const int64_t all_tiles = ((int64_t)Sk + kBN - 1) / kBN;
        g.n_split = (int)(all_tiles < want ? (all_tiles > 0 ? all_tiles : 1) : want);
    }
    g.n_wg = per * g.n_split;
    g.workspace_bytes = (size_t)heads * g.n_split * g.rows * (D + 2) * sizeof(float);
    return g;
}

hipError_t launch_decode(const AttnArgs &a, const DecodeGrid &g, void *workspace,
                         hipStream_t stream, const PagedKV *paged, int32_t *stats)
{
    if (g.n_wg == 0)
        return hipSuccess;
    DecodeParams p;
    p.a = a;
    p.rows = g.rows;
    p.n_split = g.n_split;
    p.split_len = g.split_len;
    p.kend = a.causal ? min((int64_t)a.Sk, (int64_t)a.Sq - 1 + a.offset + 1) : (int64_t)a.Sk;
    if (p.kend < 0)
        p.kend = 0;
    p.block_table = paged ? paged->block_table : nullptr;
    p.seq_lens = paged ? paged->seq_lens : nullptr;
    p.max_pages = paged ? paged->max_pages : 0;
    p.n_pages = paged ? paged->n_pages : 0;
    p.part = (float *)workspace;
    p.stats = stats;
    if (a.D == 128) {
        if (a.kv == KV_F16)
            return launch<128, KV_F16>(p, g.n_wg, stream);
        if (a.kv == KV_BF16)
            return launch<128, KV_BF16>(p, g.n_wg, stream);
        if (a.kv == KV_F16_Q4_0)
            return launch<128, KV_F16_Q4_0>(p, g.n_wg, stream);
        if (a.kv == KV_Q4_0_F16)
            return launch<128, KV_Q4_0_F16>(p, g.n_wg, stream);
        return launch<128, KV_Q4_0>(p, g.n_wg, stream);
    }
    if (a.kv == KV_F16)
        return launch<64, KV_F16>(p, g.n_wg, stream);
    if (a.kv == KV_BF16)
        return launch<64, KV_BF16>(p, g.n_wg, stream);
    if (a.kv == KV_F16_Q4_0)
        return launch<64, KV_F16_Q4_0>(p, g.n_wg, stream);
    if (a.kv == KV_Q4_0_F16)
        return launch<64, KV_Q4_0_F16>(p, g.n_wg, stream);
    return launch<64, KV_Q4_0>(p, g.n_wg, stream);
}

}  // namespace fa
