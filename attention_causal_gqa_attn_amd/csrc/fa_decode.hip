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

namespace {

struct DecodeParams {
    AttnArgs a;
    int rows, n_split, split_len;
    int64_t kend;          // keys any row can see: [0, kend)
    float *part;           // [B][Hkv][n_split][rows][D + 2]
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

// Combine the 4 waves' softmax states of each row (through LDS at cmb, 4*16*(D+2) floats)
// and write the split's partial [F, L, O] rows.
template <int D>
__device__ __forceinline__ void decode_combine(const DecodeParams &p, float *cmb, int b, int kvh,
                                               int s, int t, int wave, int quad, int r,
                                               const f32x4 *acc, float frame, float lsum)
{
    const AttnArgs &a = p.a;
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

    float *out = p.part + (((int64_t)b * a.Hkv + kvh) * p.n_split + s) * p.rows * (D + 2);
    for (int e = t; e < p.rows * D; e += kThreads) {
        const int rr = e / D, d = e % D;
        float F = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            F = fmaxf(F, cmb_f[w * 16 + rr]);
        float o = 0.0f, l = 0.0f;
        if (F != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sw = exp2_fast(cmb_f[w * 16 + rr] - F);   // 0 for an empty wave
                o += sw * cmb_o[(w * 16 + rr) * D + d];
                l += sw * cmb_l[w * 16 + rr];
            }
        }
        out[rr * (D + 2) + d] = o;
        if (d == 0) {
            out[rr * (D + 2) + D] = F;
            out[rr * (D + 2) + D + 1] = l;
        }
    }
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

    const int64_t ks = (int64_t)s * p.split_len;
    const int64_t ke = min(ks + p.split_len, p.kend);
    const int nb = ke > ks ? (int)((ke - ks + kBN - 1) / kBN) : 0;

    // row r = qi * G + hl; rows >= p.rows are padding
    const bool row_on = r < p.rows;
    const int qi = row_on ? r / a.G : 0;
    const int hl = row_on ? r % a.G : 0;
    const int h = kvh * a.G + hl;
    int64_t rowlim = ke - 1;                        // last key this row may see in the split
    if (a.causal)
        rowlim = min(rowlim, (int64_t)qi + a.offset);
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
        ld[u].init(a.k, a.v, (int64_t)b * a.Sk * a.Hkv + kvh, a.Hkv, a.Sk, t);
    uint16_t *lk = lds, *lv = lds + Geo::kElems;
    int kb0 = 0;
    if (nb >= 2 * NSETS) {
        // Steady state: the prologue and every iteration issue the same loads in the same
        // order, so the compiler's in-order load accounting stays exact and storing set u
        // waits only for set u, not for the sets issued after it.
#pragma unroll
        for (int u = 0; u < NSETS; ++u)
            ld[u].load((int)ks + u * kBN);
        for (; kb0 + 2 * NSETS <= nb; kb0 += NSETS) {
#pragma unroll
            for (int u = 0; u < NSETS; ++u) {
                ld[u].store(lk, lv);
                __syncthreads();
                ld[u].load((int)ks + (kb0 + u + NSETS) * kBN);
                decode_tile<D, BF>(lk, lv, (int)ks + (kb0 + u) * kBN, wave, quad, r, rowlim,
                                   a.c, qf, acc, frame, lsum);
                __syncthreads();
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < NSETS; ++u)
            if (u < nb)
                ld[u].load((int)ks + u * kBN);
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
                    ld[u].load((int)ks + (kb + NSETS) * kBN);
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

    const int64_t ks = (int64_t)s * p.split_len;
    const int64_t ke = min(ks + p.split_len, p.kend);
    const int nb = ke > ks ? (int)((ke - ks + kBN - 1) / kBN) : 0;

    const bool row_on = r < p.rows;
    const int qi = row_on ? r / a.G : 0;
    const int hl = row_on ? r % a.G : 0;
    const int h = kvh * a.G + hl;
    int64_t rowlim = ke - 1;
    if (a.causal)
        rowlim = min(rowlim, (int64_t)qi + a.offset);
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
    const int64_t head0 = ((int64_t)b * a.Sk * a.Hkv + kvh) * LD::ROWB;
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
        const uint32_t last = (uint32_t)min(kBN - 1, a.Sk - 1 - k0);
        const uint32_t stage = raw0 + (uint32_t)((kb % kRS) * 2 * RAW_T);
#pragma unroll
        for (int m = 0; m < NIW; ++m) {
            const int i = min(wave + 4 * m, NI - 1);
            const bool is_v = i >= ST;
            const uint8_t *gt = (is_v ? vg : kg) + (int64_t)k0 * grow;
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

    LD ld;
    ld.init(a.k, a.v, (int64_t)b * a.Sk * a.Hkv + kvh, a.Hkv, a.Sk, t);
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

// One wave per (b, KV head, row): log-sum-exp merge of the row's n_split partials.
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

    float F = -INFINITY;
    for (int s = lane; s < p.n_split; s += 64)
        F = fmaxf(F, base[(int64_t)s * stride + D]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        F = fmaxf(F, __shfl_xor(F, m, 64));
    float L = 0.0f;
    for (int s = lane; s < p.n_split; s += 64) {
        const float w = F == -INFINITY ? 0.0f : exp2_fast(base[(int64_t)s * stride + D] - F);
        wts[s] = w;
        L += w * base[(int64_t)s * stride + D + 1];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        L += __shfl_xor(L, m, 64);
    __syncthreads();
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;

    const int qi = rr / a.G, hl = rr % a.G;
    uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi) * a.Hq + kvh * a.G + hl) * D;
    for (int d2 = lane; d2 < D / 2; d2 += 64) {
        float o0 = 0.0f, o1 = 0.0f;
        for (int s = 0; s < p.n_split; ++s) {
            const float w = wts[s];
            o0 += w * base[(int64_t)s * stride + 2 * d2];
            o1 += w * base[(int64_t)s * stride + 2 * d2 + 1];
        }
        *(uint32_t *)(op + 2 * d2) = pack2<BF>(o0 * inv, o1 * inv);
    }
}

template <int D, int KV>
hipError_t launch(const DecodeParams &p, int64_t n_wg, hipStream_t stream)
{
    if constexpr (KV == KV_Q4_0)
        hipLaunchKernelGGL((decode_q4_kernel<D>), dim3((unsigned)n_wg), dim3(kThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, KV>), dim3((unsigned)n_wg), dim3(kThreads), 0,
                           stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t n_rows = (int64_t)p.a.B * p.a.Hkv * p.rows;
    hipLaunchKernelGGL((decode_merge_kernel<D, KV == KV_BF16>), dim3((unsigned)n_rows), dim3(64),
                       0, stream, p);
    return hipGetLastError();
}

}  // namespace

// Split choice: about 512 workgroups in all (two per CU), each split a whole number of
// 64-key tiles and at least one tile.
constexpr int64_t kTargetWorkgroups = 512;

DecodeGrid decode_grid(int B, int Hq, int Hkv, int Sq, int Sk, int D, int64_t kend, bool bound)
{
    DecodeGrid g;
    g.rows = (Hq / Hkv) * Sq;
    const int64_t heads = (int64_t)B * Hkv;
    int64_t want = heads > 0 ? (kTargetWorkgroups + heads - 1) / heads : 1;
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
    g.n_wg = heads * g.n_split;
    g.workspace_bytes = (size_t)heads * g.n_split * g.rows * (D + 2) * sizeof(float);
    return g;
}

hipError_t launch_decode(const AttnArgs &a, const DecodeGrid &g, void *workspace,
                         hipStream_t stream)
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
    p.part = (float *)workspace;
    if (a.D == 128) {
        if (a.kv == KV_F16)
            return launch<128, KV_F16>(p, g.n_wg, stream);
        if (a.kv == KV_BF16)
            return launch<128, KV_BF16>(p, g.n_wg, stream);
        return launch<128, KV_Q4_0>(p, g.n_wg, stream);
    }
    if (a.kv == KV_F16)
        return launch<64, KV_F16>(p, g.n_wg, stream);
    if (a.kv == KV_BF16)
        return launch<64, KV_BF16>(p, g.n_wg, stream);
    return launch<64, KV_Q4_0>(p, g.n_wg, stream);
}

}  // namespace fa
