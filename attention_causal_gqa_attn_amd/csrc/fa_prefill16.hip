// Prefill kernel for f16 / bf16 caches: the same flash organisation as the q4_0-capable
// kernel in fa_prefill.hip (K-ahead software pipeline, deferred rescale, S^T layout with one
// query row per lane), with the K/V tiles moved by the LDS DMA path of gfx950:
//
//  * `global_load_lds_dwordx4` writes each tile straight from global memory into LDS — no
//    staging registers — so a ring of 4 tile stages keeps two tiles in flight while one is
//    computed (the pipeline waits on explicit load counts; a bare s_barrier with a compiler
//    memory fence replaces __syncthreads, whose full fence would wait for every load);
//  * tiles keep their natural row-major [key][d] layout, with 16-byte chunks XOR-swizzled per
//    row so that the fragment reads below are bank-conflict free;
//  * K fragments (the A operand of S^T = K Q^T) are 16-byte row reads; the swizzle is chosen so
//    that the address of K-step st is (base | X) ^ 32*st — one VALU op per step;
//  * V^T fragments (the A operand of O^T += V^T P^T) come from `ds_read_b64_tr_b16`: within each
//    16-lane group, if source lane i reads V[key0 + i/4][d0 + 4*(i%4) .. +3], result lane j holds
//    V[key0 .. key0+3][d0 + j] — 4 consecutive keys of one d, two reads per MFMA operand;
//  * 8 waves per workgroup (4 heads x 64 queries for GQA 4), one workgroup per CU.
#include <cstdlib>

#include "fa_kernels.h"
#include "fa_tiles.h"

namespace fa {

namespace {

constexpr int kNW = 8;                 // waves per workgroup
constexpr int kNT = 64 * kNW;          // threads per workgroup
constexpr int kStages = 4;             // K/V tile stages in LDS

struct Prefill16Params {
    AttnArgs a;
    int hpw, qsub, n_qblk, n_hchunk;
};

// s_waitcnt immediate: wait until at most `vm` vector-memory ops are outstanding and all LDS
// ops are done (expcnt left unconstrained).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// One LDS-DMA transfer: every lane copies 16 bytes from gbase + voff into LDS at
// lds_base + 16 * lane. Issued from asm so that the compiler does not track it as an
// outstanding LDS write: it would otherwise wait for every such load (including the tiles that
// are meant to stay in flight) before each LDS read. The kernel orders the LDS data itself
// with explicit s_waitcnt vmcnt counts and barriers, and nothing else in it uses M0.
// An SALU write of M0 needs one wait state before the LDS-DMA load that reads it.
__device__ __forceinline__ void dma16(const uint8_t *gbase, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds_base) : "memory");
}

// LDS byte address of a wave-uniform pointer into the kernel's shared array, as an SGPR value
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p)
{
    const auto lp = (const __attribute__((address_space(3))) uint8_t *)p;
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lp);
}

__device__ __forceinline__ int k_row_perm16(int m)
{
    const int a = m >> 3, hh = (m >> 2) & 1, bb = m & 3;
    return ((a >> 1) << 4) | (hh << 3) | ((a & 1) << 2) | bb;
}

template <int D>
struct Geom16 {
    static constexpr int ROW = D * 2;                  // bytes per key row
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int TILE = kBN * ROW;             // bytes per K (or V) tile
    static constexpr int NDMA = TILE / (kNT * 16);     // DMA instructions per thread per tile
    static constexpr int LDS = 2 * kStages * TILE;
    // chunk swizzles: slot = chunk ^ sw(row)
    __device__ static __forceinline__ int swk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static __forceinline__ int swv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

template <int D, bool BF>
__global__ __launch_bounds__(kNT, 2) void prefill16_kernel(Prefill16Params p)
{
    using G = Geom16<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[G::LDS];
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

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

    const int bmq = 32 * p.qsub;
    const int qwg0 = qb * bmq;
    const int hs = wave % p.hpw, qs = wave / p.hpw;
    const int hl = hc * p.hpw + hs;
    const int q0 = qwg0 + qs * 32;
    const bool wave_on = (wave < p.hpw * p.qsub) && (hl < a.G) && (q0 < a.Sq);
    const int h = kvh * a.G + min(hl, a.G - 1);

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
                                  : (int64_t)a.Sk - 1;
    const int64_t klim_min = a.causal ? min((int64_t)a.Sk - 1, (int64_t)q0 + a.offset)
                                      : (int64_t)a.Sk - 1;

    // ---- Q once, as B operands ---------------------------------------------------------------
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
    float frame = -INFINITY, lsum = 0.0f;

    // ---- DMA of tiles: thread t's chunk n = (i * kNW + wave) * 64 + lane of instruction i ----
    const uint8_t *kg = (const uint8_t *)a.k + ((int64_t)b * a.Sk * a.Hkv + kvh) * G::ROW;
    const uint8_t *vg = (const uint8_t *)a.v + ((int64_t)b * a.Sk * a.Hkv + kvh) * G::ROW;
    const uint32_t grow = (uint32_t)a.Hkv * G::ROW;       // bytes between consecutive keys
    int drow[G::NDMA];
    uint32_t kcol[G::NDMA], vcol[G::NDMA];
#pragma unroll
    for (int i = 0; i < G::NDMA; ++i) {
        const int n = (i * kNW + wave) * 64 + lane;
        const int r = n / G::CPR, s = n % G::CPR;
        drow[i] = r;
        kcol[i] = (uint32_t)((s ^ G::swk(r)) * 16);
        vcol[i] = (uint32_t)((s ^ G::swv(r)) * 16);
    }
    auto kstage = [&](int tile) { return lds + (tile % kStages) * G::TILE; };
    auto vstage = [&](int tile) { return lds + (kStages + tile % kStages) * G::TILE; };
    auto dma_tile = [&](int tile) {
        const int k0 = tile * kBN;
        const int last = a.Sk - 1 - k0;
        const uint8_t *kt = kg + (int64_t)k0 * grow;
        const uint8_t *vt = vg + (int64_t)k0 * grow;
        uint8_t *ks = kstage(tile), *vs = vstage(tile);
#pragma unroll
        for (int i = 0; i < G::NDMA; ++i) {
            const uint32_t roff = (uint32_t)min(drow[i], last) * grow;
            const int wofs = (i * kNW + wave) * 1024;        // this wave's 1 KB of the tile
            dma16(kt, roff + kcol[i], lds_addr(ks + wofs));
            dma16(vt, roff + vcol[i], lds_addr(vs + wofs));
        }
    };
    // wait until at most `pending` tiles of DMA are outstanding, then synchronise the waves
    auto sync_tiles = [&](bool one_pending) {
        if (one_pending)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * G::NDMA));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        asm volatile("s_barrier" ::: "memory");
    };

    // ---- fragment addressing -----------------------------------------------------------------
    // K: row krow = hf*32 + perm(col); chunk 2*st + half; byte offset in the tile
    //    krow*ROW + 16*((2*st + half) ^ swk(krow)) = (krow*ROW | X) ^ 32*st
    const int krow0 = k_row_perm16(col);
    const uint32_t kfx = (uint32_t)(krow0 * G::ROW) | (uint32_t)(16 * (half ^ G::swk(krow0)));
    // V^T via transpose reads: group g = lane/16, position j = lane%16 as a source lane reads
    // V[16*t4 + 8*(g/2) + 4*sec + j/4][32*dt + 16*(g%2) + 4*(j%4) .. +3]
    const int g = lane >> 4, j = lane & 15;
    const int vr0 = 8 * (g >> 1) + (j >> 2);                  // row within a 16-key group
    const int vchunk = 2 * (g & 1) + ((j & 3) >> 1);          // chunk within a 32-column block
    const uint32_t vfx = (uint32_t)(vr0 * G::ROW) +
                         (uint32_t)(16 * (vchunk ^ G::swv(vr0)) + 8 * (j & 1));
    // for dt: chunk 4*dt + vchunk, swizzled: (4*dt) ^ swv only touches bits the dt term owns
    auto vread = [&](const uint8_t *vs, int t4, int dt) -> u32x4 {
        const uint32_t o = (vfx ^ (uint32_t)(64 * dt)) + (uint32_t)(16 * t4 * G::ROW);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vs + o));
        const s16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vs + o + 4 * G::ROW));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return (u32x4){l2[0], l2[1], h2[0], h2[1]};
    };
    auto scores = [&](const uint8_t *ks, f32x16 *s) {
        s[0] = (f32x16){};
        s[1] = (f32x16){};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const uint8_t *kp = ks + (kfx ^ (uint32_t)(32 * st));
            s[0] = mfma32<BF>(*(const u32x4 *)kp, qf[st], s[0]);
            s[1] = mfma32<BF>(*(const u32x4 *)(kp + 32 * G::ROW), qf[st], s[1]);
        }
    };

    // ---- prologue: tiles 0, 1, 2 in flight; wait for 0 and 1 ----------------------------------
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (i < nb)
            dma_tile(i);
    sync_tiles(nb > 2);

    f32x16 s_a[2], s_b[2];
    if (wave_on && nb > 0 && 0 < wkend)
        scores(kstage(0), s_a);

    auto tile = [&](const int kb, f32x16 *s_cur, f32x16 *s_next) {
        // tile kb+1 resident (tile kb+2 may still be in flight); every wave is past tile kb-1,
        // so its stage can be refilled with tile kb+3
        if (kb > 0)
            sync_tiles(kb + 2 < nb);
        if (kb + 3 < nb)
            dma_tile(kb + 3);
        const int k0 = kb * kBN;
        const bool do_cur = wave_on && k0 < wkend;
        const bool do_next = wave_on && kb + 1 < nb && k0 + kBN < wkend;

        if (do_cur) {
            if ((int64_t)k0 + kBN - 1 > klim_min) {
                const int lim = (int)max(min(klim - k0, (int64_t)kBN), (int64_t)-1) - 8 * half;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (hf * 32 + 16 * (i / 8) + (i % 8) > lim)
                            s_cur[hf][i] = -INFINITY;
            }
            float mx = s_cur[0][0];
#pragma unroll
            for (int i = 1; i < 16; ++i)
                mx = fmaxf(mx, s_cur[0][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s_cur[1][i]);
            mx = pair_max(mx);
            const float m2 = mx * a.c;
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

        const float fr = (frame == -INFINITY) ? 0.0f : frame;
        u32x4 pf[4];
        auto p_chunk = [&](int jj) {
            const int t4 = jj >> 2, e = jj & 3;
            const int i = 8 * (t4 & 1) + 2 * e;
            const float p0 = exp2_fast(__builtin_fmaf(s_cur[t4 >> 1][i], a.c, -fr));
            const float p1 = exp2_fast(__builtin_fmaf(s_cur[t4 >> 1][i + 1], a.c, -fr));
            const uint32_t pk = pack2<BF>(p0, p1);
            pf[t4][e] = pk;
            lsum = sum2<BF>(pk, lsum);
        };
        const uint8_t *vs = vstage(kb);
        auto pv = [&](int t4) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = mfma32<BF>(vread(vs, t4, dt), pf[t4], acc[dt]);
        };
        if (do_cur && do_next) {
            constexpr int NMF = D / 8;
            constexpr int PER = 16 / NMF;
            const uint8_t *ks = kstage(kb + 1);
            s_next[0] = (f32x16){};
            s_next[1] = (f32x16){};
#pragma unroll
            for (int jm = 0; jm < NMF; ++jm) {
                const int hf = jm & 1, st = jm >> 1;
                const uint8_t *kp = ks + (kfx ^ (uint32_t)(32 * st)) + hf * 32 * G::ROW;
                s_next[hf] = mfma32<BF>(*(const u32x4 *)kp, qf[st], s_next[hf]);
#pragma unroll
                for (int c = 0; c < PER; ++c) {
                    const int jj = jm * PER + c;
                    p_chunk(jj);
                    if ((jj & 3) == 3)
                        pv(jj >> 2);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NMF + 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
        } else {
            if (do_next)
                scores(kstage(kb + 1), s_next);
            if (do_cur) {
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    p_chunk(jj);
                    if ((jj & 3) == 3)
                        pv(jj >> 2);
                }
            }
        }
    };

    for (int kb = 0; kb < nb; kb += 2) {
        tile(kb, s_a, s_b);
        if (kb + 1 < nb)
            tile(kb + 1, s_b, s_a);
    }
    // no DMA is outstanding here: the last wait was for zero pending tiles

    // ---- epilogue ----------------------------------------------------------------------------
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

template <int D, bool BF>
hipError_t launch16(const Prefill16Params &p, int64_t n_wg, hipStream_t stream)
{
    hipLaunchKernelGGL((prefill16_kernel<D, BF>), dim3((unsigned)n_wg), dim3(kNT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill16(const AttnArgs &a, const PrefillGrid &g, hipStream_t stream)
{
    const Prefill16Params p{a, g.hpw, g.qsub, g.n_qblk, g.n_hchunk};
    if (a.D == 128)
        return a.kv == KV_BF16 ? launch16<128, true>(p, g.n_wg, stream)
                               : launch16<128, false>(p, g.n_wg, stream);
    return a.kv == KV_BF16 ? launch16<64, true>(p, g.n_wg, stream)
                           : launch16<64, false>(p, g.n_wg, stream);
}

}  // namespace fa
