// Prefill kernel: causal grouped-query flash attention on gfx950 MFMA.
//
// What it computes follows the fused SDPA prefill of the mlxcel PR #2306 ("defer SDPA
// accumulator rescale, stage Q once per block"): a loop over K blocks that forms scores,
// keeps each row's O accumulators and sum l in the softmax frame f it was last rescaled to,
// rescales only when a block maximum exceeds f by more than 10, and accumulates P.V; Q is
// staged once. The layout of the work is this kernel's own, built for CDNA4:
//
//  * one workgroup = 4 waves = 4 x 32 query rows of one KV head's group (e.g. 4 heads x 32
//    queries for GQA 32/8), so each K/V tile in LDS serves every head of the group;
//  * each wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (keys on M, its 32 query rows
//    on N). The C layout then gives every lane one query row, so the row maximum is a
//    register reduction plus one exchange with lane l^32, and the rescale factor is one
//    scalar per lane;
//  * K rows are fed to the MFMA in a permuted order chosen so that the S^T accumulator
//    registers of a lane are already the B operand (8 consecutive keys) of O^T += V^T P^T —
//    P never leaves registers;
//  * V is transposed into LDS once per tile (shared by the 4 waves), so the A operand of the
//    P.V MFMA is one 16-byte LDS read;
//  * K/V tiles are double-buffered with one barrier per tile; the next tile's global loads
//    are in flight while the current one is computed;
//  * workgroups are ordered heaviest-first for causal work and mapped so that one XCD works
//    through one KV head at a time (its L2 then serves all of that head's workgroups).
#include <cstdlib>

#include "fa_kernels.h"
#include "fa_tiles.h"

namespace fa {

namespace {

struct PrefillParams {
    AttnArgs a;
    int hpw, qsub, n_qblk, n_hchunk;
};

// Row of the K tile fed to A-operand row m (0..31) of a 32-key half, so that C register i of
// lane l holds key 16*(i/8) + 8*(l/32) + i%8 of the half.
__device__ __forceinline__ int k_row_perm(int m)
{
    const int a = m >> 3, hh = (m >> 2) & 1, bb = m & 3;
    return ((a >> 1) << 4) | (hh << 3) | ((a & 1) << 2) | bb;
}

// NW waves per workgroup (4 or 8), each 32 query rows; two workgroup-waves per SIMD.
template <int D, int KV, int NW>
__global__ __launch_bounds__(64 * NW, 2) void prefill_kernel(PrefillParams p)
{
    constexpr bool BF = (KV == KV_BF16);
    constexpr int NT = 64 * NW;
    using Geo = TileGeom<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Geo::stage];

    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int half = lane >> 5, col = lane & 31;

    // ---- which (b, kv head, head chunk, query block) this workgroup owns -------------------
    int rest = xcd_remap(blockIdx.x, gridDim.x);
    const int qbl = rest % p.n_qblk;
    rest /= p.n_qblk;
    const int hc = rest % p.n_hchunk;
    rest /= p.n_hchunk;
    const int kvh = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int qb = a.causal ? p.n_qblk - 1 - qbl : qbl;      // heaviest blocks first

    const int bmq = 32 * p.qsub;                              // queries per workgroup
    const int qwg0 = qb * bmq;
    const int hs = wave % p.hpw, qs = wave / p.hpw;
    const int hl = hc * p.hpw + hs;                           // head within the group
    const int q0 = qwg0 + qs * 32;
    const bool wave_on = (wave < p.hpw * p.qsub) && (hl < a.G) && (q0 < a.Sq);
    const int h = kvh * a.G + min(hl, a.G - 1);

    // keys the workgroup needs, and those this wave needs
    const int qlast_wg = min(qwg0 + bmq, a.Sq) - 1;
    int64_t kend = a.Sk;
    if (a.causal)
        kend = min((int64_t)a.Sk, (int64_t)qlast_wg + a.offset + 1);
    kend = max(kend, (int64_t)0);
    const int nb = (int)((kend + kBN - 1) / kBN);

    int64_t wkend = a.Sk;
    if (a.causal)
        wkend = min((int64_t)a.Sk, (int64_t)min(q0 + 31, a.Sq - 1) + a.offset + 1);
    const int qi = q0 + col;
    const int64_t klim = a.causal ? min((int64_t)a.Sk - 1, (int64_t)qi + a.offset)
                                  : (int64_t)a.Sk - 1;        // visible keys: j <= klim
    const int64_t klim_min = a.causal ? min((int64_t)a.Sk - 1, (int64_t)q0 + a.offset)
                                      : (int64_t)a.Sk - 1;

    // ---- stage this wave's Q rows once, as B operands (8 consecutive d per lane) ----------
    const int qrow = min(qi, a.Sq - 1);
    const uint16_t *qp = (const uint16_t *)a.q + (((int64_t)b * a.Sq + qrow) * a.Hq + h) * D;
    u32x4 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = *(const u32x4 *)(qp + 16 * s + 8 * half);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        settle(qf[s]);

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = (f32x16){};
    float frame = -INFINITY;     // row's softmax frame, log2 units of the scaled score
    float lsum = 0.0f;           // this lane's share of the row sum, in the frame

    // LDS: two K tiles and two V^T tiles. K is staged one tile ahead of V, so that while a
    // wave turns tile kb's scores into P (VALU), the MFMAs of tile kb+1's scores can run.
    uint16_t *const kbuf0 = lds;
    uint16_t *const vbuf0 = lds + 2 * Geo::kElems;
    auto kbuf = [&](int i) { return kbuf0 + (i & 1) * Geo::kElems; };
    auto vbuf = [&](int i) { return vbuf0 + (i & 1) * Geo::vElems; };

    TileLoader<D, KV, NT> ld;
    ld.init(a.k, a.v, (int64_t)b * a.Sk * a.Hkv + kvh, a.Hkv, a.Sk, t);
    if (nb > 0) {
        ld.load(0);
        ld.store(kbuf(0), vbuf(0));
    }
    if (nb > 1) {
        ld.load_k(kBN);
        ld.store_k(kbuf(1));
    }
    __syncthreads();

    const int krow0 = k_row_perm(col);
    // S^T of the K tile in `lk` for this wave's rows: two 32-key halves
    auto scores = [&](const uint16_t *lk, f32x16 *s) {
        const uint16_t *kr = lk + krow0 * Geo::kStride + 8 * half;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            s[hf] = (f32x16){};
#pragma unroll
            for (int st = 0; st < D / 16; ++st)
                s[hf] = mfma32<BF>(*(const u32x4 *)(kr + hf * 32 * Geo::kStride + 16 * st),
                                   qf[st], s[hf]);
        }
    };

    // One key tile: s_cur holds this tile's scores, s_next receives the next tile's. The loop
    // below is unrolled by two with the buffers swapping roles, so no scores are copied.
    auto tile = [&](const int kb, f32x16 *s_cur, f32x16 *s_next) {
        const int k0 = kb * kBN;
        const bool load_k = kb + 2 < nb, load_v = kb + 1 < nb;
        if (load_k)
            ld.load_k(k0 + 2 * kBN);
        if (load_v)
            ld.load_v(k0 + kBN);
        const bool do_cur = wave_on && k0 < wkend;
        const bool do_next = wave_on && kb + 1 < nb && k0 + kBN < wkend;

        if (do_cur) {
            // causal / sequence-end mask, only where a key can exceed the row's limit; keys are
            // compared relative to the tile start, in 32 bits
            if ((int64_t)k0 + kBN - 1 > klim_min) {
                const int lim = (int)max(min(klim - k0, (int64_t)kBN), (int64_t)-1) - 8 * half;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (hf * 32 + 16 * (i / 8) + (i % 8) > lim)
                            s_cur[hf][i] = -INFINITY;
            }
            // block maximum of the row (this lane's 32 keys, then lane l^32's)
            float mx = s_cur[0][0];
#pragma unroll
            for (int i = 1; i < 16; ++i)
                mx = fmaxf(mx, s_cur[0][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s_cur[1][i]);
            mx = pair_max(mx);
            const float m2 = mx * a.c;

            // deferred rescale: only rows whose block max outgrows the frame by the margin
            const bool need = m2 > frame + kRescaleMarginLog2;
            if (__any(need)) {
                const float alpha = need ? exp2_fast(frame - m2) : 1.0f;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    acc[dt] *= alpha;
                lsum *= alpha;
                frame = need ? m2 : frame;
            }
        }

        // This tile's P = 2^(S*c - f) (VALU) and the next tile's scores (MFMA) are independent:
        // in the common case both are written as one straight-line block, one MFMA of the
        // next scores (the two 32-key halves alternate, so consecutive MFMAs do not depend on
        // each other) between chunks of P, so the two instruction streams overlap.
        const float fr = (frame == -INFINITY) ? 0.0f : frame;
        u32x4 pf[4];
        auto p_chunk = [&](int j) {      // P pair j of 16 -> pf[j / 4][j % 4]
            const int t4 = j >> 2, e = j & 3;
            const int i = 8 * (t4 & 1) + 2 * e;
            const float p0 = exp2_fast(__builtin_fmaf(s_cur[t4 >> 1][i], a.c, -fr));
            const float p1 = exp2_fast(__builtin_fmaf(s_cur[t4 >> 1][i + 1], a.c, -fr));
            const uint32_t pk = pack2<BF>(p0, p1);
            pf[t4][e] = pk;
            lsum = sum2<BF>(pk, lsum);
        };
        // O^T += V^T P^T for the 16 keys of P fragment t4
        const uint16_t *lv = vbuf(kb);
        auto pv = [&](int t4) {
            const uint16_t *vr = lv + col * Geo::vStride + 16 * t4 + 8 * half;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = mfma32<BF>(*(const u32x4 *)(vr + 32 * dt * Geo::vStride), pf[t4],
                                     acc[dt]);
        };
        if (do_cur && do_next) {
            // one straight-line block: per step one MFMA of the next scores, one P pair, and
            // after every fourth pair the 4 P.V MFMAs of those 16 keys
            constexpr int NMF = D / 8;                 // MFMAs of one tile's scores
            constexpr int PER = 16 / NMF;              // P pairs per MFMA
            const uint16_t *kr = kbuf(kb + 1) + krow0 * Geo::kStride + 8 * half;
            s_next[0] = (f32x16){};
            s_next[1] = (f32x16){};
#pragma unroll
            for (int j = 0; j < NMF; ++j) {
                const int hf = j & 1, st = j >> 1;
                s_next[hf] = mfma32<BF>(*(const u32x4 *)(kr + hf * 32 * Geo::kStride + 16 * st),
                                        qf[st], s_next[hf]);
#pragma unroll
                for (int c = 0; c < PER; ++c) {
                    const int jj = j * PER + c;
                    p_chunk(jj);
                    if ((jj & 3) == 3)
                        pv(jj >> 2);
                }
            }
            // Instruction order for the block: 4 LDS fragment reads ahead, then repeatedly one
            // MFMA, one LDS read and three VALU ops, so that each MFMA's operand was requested
            // several MFMAs earlier and the VALU work issues while the MFMAs run.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NMF + 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
        } else {
            if (do_next)
                scores(kbuf(kb + 1), s_next);
            if (do_cur) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    p_chunk(j);
                    if ((j & 3) == 3)
                        pv(j >> 2);
                }
            }
        }
        if (load_k)
            ld.store_k(kbuf(kb));
        if (load_v)
            ld.store_v(vbuf(kb + 1));
        __syncthreads();
    };

    f32x16 s_a[2], s_b[2];
    if (wave_on && nb > 0 && 0 < wkend)
        scores(kbuf(0), s_a);
    for (int kb = 0; kb < nb; kb += 2) {
        tile(kb, s_a, s_b);
        if (kb + 1 < nb)
            tile(kb + 1, s_b, s_a);
    }

    // ---- epilogue: O / l, cast, store ----------------------------------------------------
    const float ltot = pair_sum(lsum);
    if (!wave_on || qi >= a.Sq)
        return;
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi) * a.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            u32x2 w;
            w[0] = pack2<BF>(acc[dt][4 * ii + 0] * inv, acc[dt][4 * ii + 1] * inv);
            w[1] = pack2<BF>(acc[dt][4 * ii + 2] * inv, acc[dt][4 * ii + 3] * inv);
            *(u32x2 *)(op + 32 * dt + 8 * ii + 4 * half) = w;
        }
}

template <int D, int KV, int NW>
hipError_t launch(const PrefillParams &p, int64_t n_wg, hipStream_t stream)
{
    hipLaunchKernelGGL((prefill_kernel<D, KV, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0,
                       stream, p);
    return hipGetLastError();
}

template <int NW>
hipError_t launch_waves(const PrefillParams &p, int D, int kv, int64_t n_wg, hipStream_t stream)
{
    if (D == 128) {
        if (kv == KV_F16)
            return launch<128, KV_F16, NW>(p, n_wg, stream);
        if (kv == KV_BF16)
            return launch<128, KV_BF16, NW>(p, n_wg, stream);
        return launch<128, KV_Q4_0, NW>(p, n_wg, stream);
    }
    if (kv == KV_F16)
        return launch<64, KV_F16, NW>(p, n_wg, stream);
    if (kv == KV_BF16)
        return launch<64, KV_BF16, NW>(p, n_wg, stream);
    return launch<64, KV_Q4_0, NW>(p, n_wg, stream);
}

PrefillGrid grid_for(const AttnArgs &a, int waves)
{
    PrefillGrid g;
    g.waves = waves;
    g.hpw = a.G < waves ? a.G : waves;
    g.qsub = waves / g.hpw;
    g.n_qblk = (a.Sq + 32 * g.qsub - 1) / (32 * g.qsub);
    g.n_hchunk = (a.G + g.hpw - 1) / g.hpw;
    g.n_wg = (int64_t)g.n_qblk * g.n_hchunk * a.Hkv * a.B;
    return g;
}

}  // namespace

// Workgroup size: 8 waves (the K/V tiles in LDS serve twice as many query rows, halving the
// tile traffic) when that still gives at least one workgroup per CU, else 4 waves.
// FA_PREFILL_WAVES=4|8 overrides the choice (for tuning).
PrefillGrid prefill_grid(const AttnArgs &a)
{
    if (a.kv != KV_Q4_0)
        return prefill16_grid(a);
    static const int forced = [] {
        const char *e = getenv("FA_PREFILL_WAVES");
        return e ? atoi(e) : 0;
    }();
    if (forced == 4 || forced == 8)
        return grid_for(a, forced);
    const PrefillGrid g8 = grid_for(a, 8);
    return g8.n_wg >= 256 ? g8 : grid_for(a, 4);
}

hipError_t launch_prefill(const AttnArgs &a, hipStream_t stream)
{
    const PrefillGrid g = prefill_grid(a);
    const PrefillParams p{a, g.hpw, g.qsub, g.n_qblk, g.n_hchunk};
    if (g.n_wg == 0)
        return hipSuccess;
    if (a.kv != KV_Q4_0)
        return launch_prefill16(a, g, stream);
    if (g.waves == 8)
        return launch_waves<8>(p, a.D, a.kv, g.n_wg, stream);
    return launch_waves<4>(p, a.D, a.kv, g.n_wg, stream);
}

}  // namespace fa
