// Prefill kernel for f16 / bf16 caches: flash attention with the S^T = K Q^T layout (one query
// row per lane), the deferred O/l rescale, and K/V tiles moved into LDS by the LDS-DMA path of
// gfx950. Organisation, chosen from measurement on the chip:
//
//  * 4 waves per workgroup, one per SIMD, 64 query rows per wave as two 32-row blocks (j = 0, 1)
//    of one head: every K or V^T fragment read from LDS feeds two MFMAs, halving the LDS read
//    traffic against 32 rows per wave (the 2-byte transpose read runs at half the LDS rate of
//    a 16-byte read, and LDS bandwidth is what 32-row waves run out of);
//  * one wave per SIMD has to overlap its own softmax VALU work with its MFMAs. A 32x32x16 MFMA
//    keeps the issue port busy for half of its 32 cycles, so each one leaves room for a few
//    VALU instructions; a steady-state tile is written as a fixed sequence of MFMA slots with
//    the softmax work spread over them, and scheduling barriers keep that order:
//        half 1 of tile n:  acc[j] += V(n-1)^T P(n-1, j)^T, both blocks    | softmax(n, j = 0)
//        half 2 of tile n:  S(n+1, j) = K(n+1) Q(j)^T, both blocks          | softmax(n, j = 1)
//    (block 1's scores are double-buffered: its softmax reads S(n) while S(n+1) is written);
//  * tiles keep their row-major [key][d] layout in LDS with 16-byte chunks XOR-swizzled per
//    row, so K fragment reads (16 bytes) and V^T transpose reads (ds_read_b64_tr_b16) are free
//    of bank conflicts; K runs 4 tiles ahead of its use and V 2 tiles, through 4-stage rings,
//    so every tile has three loop iterations to arrive (16-bit caches at D = 64: 8-stage rings,
//    K 7 tiles ahead and V 5, and one barrier per pair of tiles);
//  * a q4_0 cache arrives raw (12-byte LDS-DMA chunks, K 4 tiles and V 2 tiles ahead) and the
//    waves dequantize it into 2-stage f16 K and V rings of the same layout, one tile of each per
//    iteration (K two tiles ahead of its scores, V one ahead of its P.V), so everything after
//    the dequantization is the f16 kernel; with one q4_0 and one f16 cache (mixed K/V types)
//    the f16 tensor keeps the direct 4-stage ring and only the q4_0 one takes the raw path;
//  * a paged cache (64-key pages, a block table and per-sequence lengths) differs only in where
//    a tile's bytes start and where a sequence ends: the workgroup copies its sequence's page
//    numbers into LDS once, and each iteration reads the two it needs (K n+4, V n+2) at its
//    start, before the slots that issue the transfers.
#include <cstdlib>
#include <utility>

#include <algorithm>

#include "fa_kernels.h"
#include "fa_tiles.h"

namespace fa {

namespace {

// every helper lambda of the kernel is inlined: the kernel relies on scalar (wave-uniform)
// values staying scalar, and on register arrays staying registers
#define INL __attribute__((always_inline))

constexpr int kNW = 4;                 // waves per workgroup
constexpr int kNT = 64 * kNW;          // threads per workgroup
constexpr int kQW = 64;                // query rows per wave
constexpr int kStages = 4;             // tile stages per ring (K ring, V ring)

struct Prefill16Params {
    AttnArgs a;
    int hpw, qsub, n_qblk, n_hchunk;
    // paged caches only (see PagedKV); q_lens may be null (Sq queries in every sequence)
    const int32_t *block_table, *seq_lens, *q_lens;
    int max_pages, n_pages;
    // balanced causal prefill (SPLIT instances): the units (b, kv head, head chunk, query block)
    // of query block >= q_split hold more than `cap` tiles and run only their tiles [0, cap);
    // the workgroup of the mirror unit (query block n_qblk - 1 - q) runs the rest after its
    // own unit, and the two parts of a unit are merged through the workspace. n_main: the
    // workgroups (one per unit); n_tail: the split units
    int q_split, cap, n_main, n_tail;
    uint32_t *cnt;     // arrival counters, one per split unit, zero between calls
    float *part;       // partial rows [split unit][part][wave][64 rows][kPartRow floats]
    // key split (SPLIT instances with parts > 0, for shapes with few units): every unit's tiles
    // are cut into `parts` runs, one workgroup each; each writes its partial rows to
    // part[unit][run][wave][64 rows][kPartRow] and prefill_parts_merge_kernel combines them
    int parts;
    // STATS instances: per query row (b, i, h), two int32 counters written in the epilogue:
    // how many times the row's softmax frame moved (the deferred-rescale test fired for the
    // row, counting the first frame), and in how many tiles its wave block ran the O rescale
    int32_t *stats;
};
// a partial row: D unnormalised outputs, frame, sum, padding to 16 bytes
constexpr int kPartRow = 132;

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

// The same transfer with its LDS base formed as lds_a + lds_b straight into M0 and the lane's
// offset clamped to at most `lim` on the way (the clamp also provides the wait state after the
// M0 write).
__device__ __forceinline__ void dma16c(const uint8_t *gbase, uint32_t voff, uint32_t lim,
                                       uint32_t lds_a, uint32_t lds_b)
{
    uint32_t t;
    asm volatile("s_add_u32 m0, %3, %4\n\tv_min_u32 %0, %2, %1\n\tglobal_load_lds_dwordx4 %0, %5"
                 : "=&v"(t) : "v"(voff), "s"(lim), "s"(lds_a), "s"(lds_b), "s"(gbase)
                 : "memory", "scc");
}

// The 12-byte transfer with the lane's offset formed on the way, min(rowoff, lim) + col (the
// row clamped, the column kept), and its LDS base lds_a + lds_b written straight into M0.
__device__ __forceinline__ void dma12c(const uint8_t *gbase, uint32_t rowoff, uint32_t lim,
                                       uint32_t col, uint32_t lds_a, uint32_t lds_b)
{
    uint32_t t;
    asm volatile("s_add_u32 m0, %4, %5\n\tv_min_u32 %0, %2, %1\n\tv_add_u32 %0, %0, %3\n\t"
                 "global_load_lds_dwordx3 %0, %6"
                 : "=&v"(t) : "v"(rowoff), "s"(lim), "v"(col), "s"(lds_a), "s"(lds_b), "s"(gbase)
                 : "memory", "scc");
}

// One 12-byte LDS-DMA transfer per lane: gbase + voff -> LDS lds_base + 16 * lane (a 16-byte
// slot per lane), for the q4_0 rows, whose 18-byte blocks split into 12-byte chunks.
__device__ __forceinline__ void dma12(const uint8_t *gbase, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds_base) : "memory");
}

// Keeps a value's computation at this point of the instruction stream: the empty volatile asm
// cannot move across the scheduling fences, so neither can the code that produces its input.
template <typename T>
__device__ __forceinline__ void pin(T &x)
{
    asm volatile("" : "+v"(x));
}

// Score MFMAs, issued from asm so that their results land in VGPRs (the compiler would put
// every MFMA result of this kernel in AGPRs, and the softmax reads the scores with VALU
// instructions, which cannot take AGPR operands). The compiler does not see these as MFMAs:
// the kernel waits out the MFMA-to-VALU dependency itself (s_nop before the first VALU read
// of a tile's scores), and the chains accumulate in place (srcC == vdst). The Q operand is
// taken from AGPRs, where Q stays for the whole kernel. The asm is volatile: a plain asm
// statement may be moved past the scheduling fences (its order is free in the compiler's
// view), which drew half 2's softmax units and transfers in front of its first MFMA.
template <bool BF>
__device__ __forceinline__ void smfma_first(f32x16 &d, const u32x4 &a, const u32x4 &b)
{
    if constexpr (BF)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
template <bool BF>
__device__ __forceinline__ void smfma_acc(f32x16 &d, const u32x4 &a, const u32x4 &b)
{
    if constexpr (BF)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// Wait states between the score MFMAs and VALU reads of their results (a 16-pass XDL result
// needs at most 19 before a VALU reads it); each s_nop 7 gives 8. Taking the score registers
// as operands makes every later read of them depend on the wait.
__device__ __forceinline__ void smfma_drain()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
__device__ __forceinline__ void smfma_drain(f32x16 &a, f32x16 &b, f32x16 &c, f32x16 &d)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// LDS byte address of a pointer into the kernel's shared array
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p)
{
    const auto lp = (const __attribute__((address_space(3))) uint8_t *)p;
    return (uint32_t)(uintptr_t)lp;
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
    static constexpr int NDMA = TILE / (kNT * 16);     // DMA transfers per thread per tile
    static constexpr int LDS = 2 * kStages * TILE;
    // chunk swizzles: slot = chunk ^ sw(row)
    __device__ static __forceinline__ int swk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static __forceinline__ int swv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// q4_0 caches: a key row of one KV head (D/32 blocks of 18 bytes) is CPR 12-byte chunks, each
// landing in a 16-byte LDS slot (row r's chunk c in slot r * CPR + c); K raw tiles run 4 tiles
// ahead through KR stages, V 2 tiles through VR; the f16 K and V rings have 2 stages each.
template <int D>
struct Q4Raw {
    static constexpr int ROWB = 18 * (D / 32);         // bytes of a key row
    static constexpr int CPR = ROWB / 12;
    static constexpr int RAWT = kBN * CPR * 16;        // one tensor's raw tile in LDS
    static constexpr int NX = CPR;                     // wave-wide transfers per tensor tile
    static constexpr int NIW = (2 * NX + kNW - 1) / kNW;   // per wave per iteration, K + V
    static constexpr int NIW1 = (NX + kNW - 1) / kNW;      // the same for one tensor
    static constexpr int KR = 4, VR = 3;
    static constexpr int LDS = 4 * Geom16<D>::TILE + (KR + VR) * RAWT;
};

// f(std::integral_constant<int, I>) for I = B .. E-1, expanded at compile time
template <int B, typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, B + Is>{}), ...);
}
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (E > B)
        static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
}

// ---- compile-time placement of the softmax work over the MFMA slots of a tile ---------------
// A tile is 2*NM MFMA slots: slots [0, NM) are half 1 (P.V), [NM, 2*NM) half 2 (scores). The
// softmax of each block j is cut into short units:
//   M0..M7  partial maxima of the 32 scores (m8[i] = max of 4: v_max3 + v_max)
//   T1, T2  the rest of the lane's max;  P  the lane-pair max (the row max)
//   F1, F2  frame update: alpha, new frame, lsum *= alpha, whether any lane rescales
//   E0..E15 two scores to P values (exp2(s*c - frame)); Cu packs E u's pair into P chunk
//           t4 = u/4 (slot e = u%4) and adds it to lsum
// A list scheduler places them: every unit after the units it depends on (in an earlier
// slot: the slot's MFMA covers the latency), not before its earliest slot, within a cycle
// budget per slot (issue cycles of its VALU instructions; an MFMA leaves about 16 of its 32).
// Earliest slots: C units of block 0 write pf[0][t4], which the block-0 P.V MFMAs of chunk t4
// read in half 1 (the last one in slot 2*(t4*NDT + NDT - 1)); block 1's C units write
// pf[1][t4] (read up to slot 2*(t4*NDT + NDT - 1) + 1). Deadlines, checked below: block 0's
// E units for chunks 2, 3 read its hf = 1 scores, which the block-0 score MFMAs of hf = 1
// overwrite from slot NM + 2*NST on (those of chunks 0, 1, hf = 0, from slot NM).
enum UnitKind { UM, UT1, UT2, UP, UF1, UF2, UE, UC };
struct Unit {
    int j, kind, idx;
};
constexpr int kUnitsPerBlock = 8 + 5 + 16 + 16;
constexpr int kNU = 2 * kUnitsPerBlock;
constexpr int unit_cost(int kind)
{
    switch (kind) {
    case UM: return 8;
    case UT1: return 12;
    case UT2: return 4;
    case UP: return 24;
    case UF1: return 12;
    case UF2: return 28;
    case UE: return 26;
    default: return 8;
    }
}
struct Schedule {
    Unit unit[kNU];           // in slot order
    int slot[kNU];            // slot of unit[i]
    int first[129];           // units [first[s], first[s+1]) run in slot s; first[2*NM]: after
};
template <int NDT, int NST, int NM, int BUDGET>
constexpr Schedule make_schedule()
{
    // priority order
    Unit u[kNU] = {};
    int n = 0;
    auto chain = [&](int j) {
        for (int i = 0; i < 8; ++i)
            u[n++] = Unit{j, UM, i};
        u[n++] = Unit{j, UT1, 0};
        u[n++] = Unit{j, UT2, 0};
        u[n++] = Unit{j, UP, 0};
        u[n++] = Unit{j, UF1, 0};
        u[n++] = Unit{j, UF2, 0};
    };
    auto expc = [&](int j, int lo, int hi) {       // E lo..hi-1, each C one E behind
        for (int e = lo; e < hi; ++e) {
            u[n++] = Unit{j, UE, e};
            if (e > lo)
                u[n++] = Unit{j, UC, e - 1};
        }
        u[n++] = Unit{j, UC, hi - 1};
    };
    chain(0);
    expc(0, 0, 8);
    chain(1);
    expc(0, 8, 16);
    expc(1, 0, 16);
    auto earliest = [&](const Unit &x) {
        if (x.kind == UC) {
            const int t4 = x.idx / 4;
            return 2 * (t4 * NDT + NDT - 1) + 1 + x.j;
        }
        if (x.j == 1 && x.kind == UE)
            return NM;
        return 0;
    };
    // dependencies: index of each unit's predecessor(s) in u[]
    auto find = [&](int j, int kind, int idx) {
        for (int i = 0; i < kNU; ++i)
            if (u[i].j == j && u[i].kind == kind && u[i].idx == idx)
                return i;
        return -1;
    };
    int placed[kNU] = {};
    for (int i = 0; i < kNU; ++i)
        placed[i] = -1;
    Schedule sc{};
    int out = 0;
    const int budget = BUDGET;
    for (int s = 0; s < 2 * NM; ++s) {
        sc.first[s] = out;
        int room = budget;
        for (int i = 0; i < kNU; ++i) {
            if (placed[i] >= 0 || earliest(u[i]) > s)
                continue;
            const Unit &x = u[i];
            bool ready = true;
            auto need = [&](int k) {
                if (k < 0 || placed[k] < 0 || placed[k] >= s)
                    ready = false;
            };
            if (x.kind == UT1)
                for (int m = 0; m < 8; ++m)
                    need(find(x.j, UM, m));
            if (x.kind == UT2)
                need(find(x.j, UT1, 0));
            if (x.kind == UP)
                need(find(x.j, UT2, 0));
            if (x.kind == UF1)
                need(find(x.j, UP, 0));
            if (x.kind == UF2)
                need(find(x.j, UF1, 0));
            if (x.kind == UE)
                need(find(x.j, UF2, 0));
            if (x.kind == UC)
                need(find(x.j, UE, x.idx));
            if (!ready)
                continue;
            const int c = unit_cost(x.kind);
            if (c > room && room < budget)
                continue;
            room -= c;
            placed[i] = s;
            sc.unit[out] = x;
            sc.slot[out] = s;
            ++out;
            if (room <= 0)
                break;
        }
    }
    sc.first[2 * NM] = out;
    // anything left runs after the last slot, in priority order
    for (int i = 0; i < kNU; ++i)
        if (placed[i] < 0) {
            sc.unit[out] = u[i];
            sc.slot[out] = 2 * NM;
            ++out;
        }
    return sc;
}
// checks: block 0's E units meet their deadlines (the score MFMAs of half 2 overwrite the
// scores they read), and only block 1 units run after the last slot
template <int NDT, int NST, int NM>
constexpr bool schedule_ok(const Schedule &sc)
{
    for (int i = 0; i < kNU; ++i) {
        const Unit &x = sc.unit[i];
        if (x.j == 0 && x.kind == UE) {
            const int deadline = (x.idx / 8) == 0 ? NM : NM + 2 * NST;   // hf of chunk idx/4
            if (sc.slot[i] >= deadline)
                return false;
        }
        if (x.j == 0 && sc.slot[i] >= 2 * NM)
            return false;
    }
    return true;
}

template <int D>
struct Plans {
    static constexpr int NDT = D / 32;                 // 32-wide d blocks of O^T
    static constexpr int NST = D / 16;                 // k-steps of a score chain
    static constexpr int NM = 8 * NDT;                 // MFMA slots per half
    static_assert(NM == 4 * NST && NM <= 64, "both halves have NM MFMA slots");
    // VALU cycles per slot: an MFMA slot leaves about 16; D = 64 has half the MFMAs for the
    // same softmax work and packs the units tighter
    static constexpr Schedule sc = make_schedule<NDT, NST, NM, D == 128 ? 24 : 56>();
    static_assert(schedule_ok<NDT, NST, NM>(sc), "softmax units placed in time");
};

template <int D, int KT, int VT, bool PAGED, bool SPLIT = false, bool STATS = false>
__global__ __launch_bounds__(kNT, 1) void prefill16_kernel(Prefill16Params p)
{
    static_assert(!SPLIT || !PAGED, "split: contiguous caches");
    static_assert(!STATS || (!SPLIT && !PAGED), "counters: the plain contiguous kernel");
    static_assert(KT == VT || (KT != KV_BF16 && VT != KV_BF16), "bf16 caches are not mixed");
    constexpr bool BF = KT == KV_BF16;
    constexpr bool QK = KT == KV_Q4_0, QV = VT == KV_Q4_0;     // which tensors arrive raw
    constexpr bool Q4 = QK && QV, ANYQ = QK || QV;
    using G = Geom16<D>;
    using QR = Q4Raw<D>;
    using PL = Plans<D>;
    constexpr int NDT = PL::NDT, NST = PL::NST, NM = PL::NM;
    // PAIR (16-bit caches at D = 64, whose 8 KB tiles leave room for 8-stage rings): K runs 7
    // tiles ahead and V 5, and only even iterations wait and meet at a barrier, which halves
    // the barriers of a tile with half the MFMA work of D = 128
    constexpr bool PAIR = D == 64 && !ANYQ;
    constexpr int LK = PAIR ? 7 : 4, LV = PAIR ? 5 : 2;      // tiles ahead: K, V
    // f16 K and V rings (2 stages for a tensor that arrives raw, else 4 or 8), then the raw
    // rings
    constexpr int FS16 = PAIR ? 8 : kStages;
    constexpr int FSK = QK ? 2 : FS16, FSV = QV ? 2 : FS16;
    constexpr int RAW0 = (FSK + FSV) * G::TILE;
    constexpr int LDSB = RAW0 + ((QK ? QR::KR : 0) + (QV ? QR::VR : 0)) * QR::RAWT;
    static_assert(!Q4 || LDSB == QR::LDS, "q4_0 layout");
    static_assert(ANYQ || PAIR || LDSB == G::LDS, "16-bit layout");
    // transfers per wave per iteration: K(n+4) then V(n+2)
    constexpr int TK = QK ? QR::NIW1 : G::NDMA, TV = QV ? QR::NIW1 : G::NDMA;
    constexpr int TI = Q4 ? QR::NIW : TK + TV;
    static_assert(4 * TI <= NM, "every transfer has a slot");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDSB];
    __shared__ int32_t ptab[PAGED ? kPrefillMaxPages : 1];     // the sequence's page numbers
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: scalar branches
    const int half = lane >> 5, col = lane & 31;

    // ---- which (b, kv head, head chunk, query block) this workgroup owns -------------------
    int rest = xcd_remap(blockIdx.x, gridDim.x);
    int run_id = 0;                       // key split: this workgroup's run of its unit's tiles
    if constexpr (SPLIT) {
        if (p.parts > 0) {
            run_id = rest % p.parts;
            rest /= p.parts;
        }
    }
    const int unit_id = rest;             // ((b * Hkv + kvh) * n_hchunk + hc) * n_qblk + qbl
    const int qbl = rest % p.n_qblk;
    rest /= p.n_qblk;
    const int hc = rest % p.n_hchunk;
    rest /= p.n_hchunk;
    // Each XCD takes a contiguous range of these units. Contiguous caches: sequence-major. A
    // paged batch's sequences differ in length, so there the KV head is the outer index: each
    // XCD then works on one KV head of every sequence rather than on whole sequences (one
    // long sequence among short ones would otherwise run on a quarter of the chip), and all
    // query blocks of a (sequence, KV head) still share one XCD's L2. Timed on an MI355X
    // (same outputs): 4 sequences of 8192 keys with 1024, 128, 2048 and 64 queries 467 against
    // 842 us, 8 sequences of 512-4096 keys with 512 queries each 181 against 234, equal
    // sequences unchanged.
    const int kvh = PAGED ? rest / a.B : rest % a.Hkv;
    const int b = PAGED ? rest % a.B : rest / a.Hkv;
    const int qblk0 = a.causal ? p.n_qblk - 1 - qbl : qbl;    // heaviest blocks first
    __shared__ uint32_t arrived;                                // SPLIT: arrival flag

    // One unit's tiles: all of them, or (SPLIT, a split unit) its first cap tiles (part 0) or
    // the rest (part 1). The body below, down to the end of the epilogue, keeps the kernel's
    // indentation.
    auto run = [&](const int qblk, const int part) INL {
    // this sequence's keys and queries, and the position of its first query
    int sk = a.Sk, sq = a.Sq;
    int64_t off = a.offset;
    if constexpr (PAGED) {
        sk = min(max(p.seq_lens[b], 0), p.max_pages * kBN);
        sq = p.q_lens ? min(max(p.q_lens[b], 0), a.Sq) : a.Sq;
        off = (int64_t)sk - sq;
    }

    const int bmq = kQW * p.qsub;
    const int qwg0 = qblk * bmq;
    if (PAGED && qwg0 >= sq)
        return;                                  // whole workgroup: no row of it exists
    const int hs = wave % p.hpw, qs = wave / p.hpw;
    const int hl = hc * p.hpw + hs;
    const int q0 = qwg0 + qs * kQW;
    const bool wave_on = (wave < p.hpw * p.qsub) && (hl < a.G) && (q0 < sq);
    const int h = kvh * a.G + min(hl, a.G - 1);

    const int qlast_wg = min(qwg0 + bmq, sq) - 1;
    int64_t kend = sk;
    if (a.causal)
        kend = min((int64_t)sk, (int64_t)qlast_wg + off + 1);
    kend = max(kend, (int64_t)0);
    // this workgroup's tiles: [t0, t0 + nb) of the unit's
    const int nb_unit = (int)((kend + kBN - 1) / kBN);
    int t0 = 0, nb = nb_unit;
    const bool split_unit = SPLIT && qblk >= p.q_split;
    if constexpr (SPLIT) {
        if (p.parts > 0) {
            const int per = (nb_unit + p.parts - 1) / p.parts;
            t0 = run_id * per;
            nb = max(min(per, nb_unit - t0), 0);
        }
    }
    if (split_unit) {
        if (part == 0) {
            nb = min(nb_unit, p.cap);
        } else {
            t0 = p.cap;
            nb = max(nb_unit - p.cap, 0);
        }
    }

    // per block: this lane's row, its last visible key, and the block's most limited row's
    int qi[2];
    int64_t klim[2], klim_min[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        qi[j] = q0 + 32 * j + col;
        klim[j] = a.causal ? min((int64_t)sk - 1, (int64_t)qi[j] + off) : (int64_t)sk - 1;
        klim_min[j] = a.causal ? min((int64_t)sk - 1, (int64_t)(q0 + 32 * j) + off)
                               : (int64_t)sk - 1;
    }

    // ---- Q once, as B operands: qf[j][st] = row qi[j], d = 16 st + 8 half .. + 7 -----------
    u32x4 qf[2][NST];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int qrow = min(qi[j], a.Sq - 1);
        const uint16_t *qp = (const uint16_t *)a.q + (((int64_t)b * a.Sq + qrow) * a.Hq + h) * D;
#pragma unroll
        for (int s = 0; s < NST; ++s)
            qf[j][s] = *(const u32x4 *)(qp + 16 * s + 8 * half);
    }
    // Q moves to AGPRs here, once, and stays there: the score MFMAs read it from asm, and the
    // drain below separates the AGPR writes from the first MFMA that reads them
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < NST; ++s)
            asm volatile("" : "+a"(qf[j][s]));
    smfma_drain();

    f32x16 acc[2][NDT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            acc[j][dt] = (f32x16){};
    float frame[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.0f, 0.0f};
    float fr[2] = {0.0f, 0.0f}, alpha[2] = {1.0f, 1.0f};
    bool rescale[2] = {false, false};
    int nmove[2] = {0, 0}, nresc[2] = {0, 0};        // STATS counters

    // ---- tile DMA: transfer i of thread t moves 16-byte chunk n = (i*kNW + wave)*64 + lane ---
    // (b, kv head)'s key 0; a paged cache: kv head's row in a page, pages added per tile
    const int64_t hrow = PAGED ? kvh : (int64_t)b * a.Sk * a.Hkv + kvh;
    const uint8_t *kg = (const uint8_t *)a.k + hrow * G::ROW;
    const uint8_t *vg = (const uint8_t *)a.v + hrow * G::ROW;
    const uint32_t grow = (uint32_t)a.Hkv * G::ROW;       // bytes between consecutive keys
    const uint32_t lds0 = lds_addr(lds);
    // chunk (row r, column chunk c) of transfer i; K and V chunks land swizzled
    auto chunk_r = [&](int i) INL { return ((i * kNW + wave) * 64 + lane) / G::CPR; };
    auto chunk_c = [&](int i) INL { return ((i * kNW + wave) * 64 + lane) % G::CPR; };
    auto kcol = [&](int i) INL { return (uint32_t)((chunk_c(i) ^ G::swk(chunk_r(i))) * 16); };
    auto vcol = [&](int i) INL { return (uint32_t)((chunk_c(i) ^ G::swv(chunk_r(i))) * 16); };
    uint32_t rowg[G::NDMA], kc[G::NDMA], vc[G::NDMA], lwave[G::NDMA];
#pragma unroll
    for (int i = 0; i < G::NDMA; ++i) {
        rowg[i] = (uint32_t)chunk_r(i) * grow;
        kc[i] = kcol(i);
        vc[i] = vcol(i);
        lwave[i] = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((i * kNW + wave) * 1024));
    }
    // K stages [0, FSK), V stages [FSK, FSK + FSV), then the raw stages; tile j lives in K
    // stage j % FSK and V stage j % FSV
    auto kstage = [&](int tl) INL { return lds + (tl & (FSK - 1)) * G::TILE; };
    auto vstage = [&](int tl) INL { return lds + (FSK + (tl & (FSV - 1))) * G::TILE; };
    // Where tile tl sits, in tiles of kBN keys from the (b, kv head) base: tl itself, or its
    // page. Tiles past the last one re-read the last tile (into a stage nobody reads any more),
    // so every loop iteration issues the same transfers and the wait counts stay fixed.
    if constexpr (PAGED) {
        const int32_t *bt = p.block_table + (int64_t)b * p.max_pages;
        for (int i = t; i < nb; i += kNT)
            ptab[i] = min(max(bt[i], 0), p.n_pages - 1);
        __syncthreads();
    }
    auto slot = [&](int tl) INL -> int {
        tl = min(tl, nb - 1);
        if constexpr (PAGED)
            return __builtin_amdgcn_readfirstlane(ptab[tl]);
        else
            return t0 + tl;
    };
    // Transfer i of tile tl (at slot sl) of K (is_v false) or V into a stage; rows past the end
    // of the sequence repeat its last key.
    auto dma_one = [&](bool is_v, int stage, int tl, int sl, int i) INL {
        tl = min(tl, nb - 1);
        const int k0 = (t0 + tl) * kBN;
        const uint8_t *gt = (is_v ? vg : kg) + (int64_t)sl * kBN * grow;
        const uint32_t lastg = (uint32_t)min(kBN - 1, sk - 1 - k0) * grow;
        dma16(gt, min(rowg[i], lastg) + (is_v ? vc[i] : kc[i]),
              lwave[i] + (uint32_t)(stage * G::TILE));
    };
    // 16-bit caches (no raw tensor): the same transfers with less per-tile arithmetic. A lane's
    // offsets within a tile are fixed (koff, voff); the first rows of the tiles this iteration
    // reads (kcur, vcur) advance by one tile per iteration up to the last tile (a paged cache:
    // the tile's page, looked up per iteration); on the last tile, offsets past the sequence's
    // last row (tail_lim) are clamped to that row's last chunk, so every byte read lies in the
    // cache and is finite (those rows are keys every query masks, so what lands there is never
    // used).
    constexpr bool FAST16 = !ANYQ;
    // where the transfers go: at D = 128 K's in half 1 and V's in half 2 (the K fragment reads
    // of half 2 then share the LDS with half the transfers); at D = 64 all in half 2 (timed on
    // an MI355X: 0.7 % faster at D = 128, 0.5 % slower at D = 64)
    constexpr int kDmaMode = D == 128 ? 2 : 0;
    const int64_t tstep = (int64_t)kBN * grow;
    uint32_t koff[G::NDMA], voff[G::NDMA];
#pragma unroll
    for (int i = 0; i < G::NDMA; ++i) {
        koff[i] = rowg[i] + kc[i];
        voff[i] = rowg[i] + vc[i];
    }
    const uint32_t tail_lim = nb > 0
        ? (uint32_t)min((int64_t)kBN - 1, (int64_t)sk - 1 - (int64_t)(t0 + nb - 1) * kBN) * grow +
              (uint32_t)(G::ROW - 16)
        : ~0u;
    auto tile_row0 = [&](const uint8_t *base, int tl) INL {
        return base + (int64_t)(t0 + min(tl, nb - 1)) * tstep;
    };
    const uint8_t *kcur = tile_row0(kg, LK), *vcur = tile_row0(vg, LV);
    // transfer i (< NDMA: K(n+LK), else V(n+LV)) of iteration n, into the stage of K(n+LK-FSK)
    // or V(n+LV-FSV), whose last reader ran before the latest barrier; a paged cache's tiles
    // sit in pages sk4 (K) and sv2 (V)
    auto dma_fast = [&](int n, int i, int sk4, int sv2) INL {
        const bool is_v = i >= G::NDMA;
        const int ii = is_v ? i - G::NDMA : i;
        const int tl = n + (is_v ? LV : LK);
        const uint32_t lim = tl >= nb - 1 ? tail_lim : ~0u;
        const uint32_t st = (uint32_t)((is_v ? FSK + (tl & (FSV - 1)) : (tl & (FSK - 1))) * G::TILE);
        const uint8_t *src = PAGED || ANYQ
                                 ? (is_v ? vg : kg) + (int64_t)(is_v ? sv2 : sk4) * tstep
                                 : (is_v ? vcur : kcur);
        dma16c(src, is_v ? voff[ii] : koff[ii], lim, lwave[ii], st);
    };
    // after iteration n's transfers: the tiles of iteration n + 1
    auto dma_advance = [&](int n) INL {
        if constexpr (!PAGED) {
            kcur += n + LK + 1 <= nb - 1 ? tstep : 0;
            vcur += n + LV + 1 <= nb - 1 ? tstep : 0;
        }
    };

    // ---- q4_0: raw transfers and the dequantization into the f16 rings ----------------------
    const uint32_t growq = (uint32_t)a.Hkv * QR::ROWB;
    const uint8_t *kq = (const uint8_t *)a.k + hrow * QR::ROWB;
    const uint8_t *vq = (const uint8_t *)a.v + hrow * QR::ROWB;
    auto rawk = [&](int tl) INL { return lds + RAW0 + (tl & (QR::KR - 1)) * QR::RAWT; };
    auto rawv = [&](int tl) INL {
        return lds + RAW0 + (QK ? QR::KR * QR::RAWT : 0) + (tl % QR::VR) * QR::RAWT;
    };
    // transfer x of raw tile tl at slot ts (LDS slots 64 x .. 64 x + 63); tiles past the last
    // re-read the last one, rows past the sequence's end repeat its last key
    auto dma_raw = [&](bool is_v, int tl, int ts, int x) INL {
        const uint8_t *stg = is_v ? rawv(tl) : rawk(tl);
        tl = min(tl, nb - 1);
        const int64_t k0 = (int64_t)(t0 + tl) * kBN;
        const int sl = 64 * x + lane;
        const int last = (int)min((int64_t)kBN - 1, (int64_t)sk - 1 - k0);
        const uint32_t row = (uint32_t)min(sl / QR::CPR, last);
        dma12((is_v ? vq : kq) + (int64_t)ts * kBN * growq,
              row * growq + 12u * (uint32_t)(sl % QR::CPR),
              __builtin_amdgcn_readfirstlane(lds_addr(stg) + (uint32_t)(1024 * x)));
    };
    // Both tensors raw: this wave's m-th transfer of every iteration is transfer
    // i = min(wave + 4 m, 2 NX - 1) of the pair (i < NX: column i of raw K(n+4), else column
    // i - NX of raw V(n+2)), so its tensor, row offset, column and LDS column are fixed; per
    // tile only the tile's base, the row limit and the stage change
    constexpr int NIWQ = Q4 ? QR::NIW : 1;
    uint32_t rq_off[NIWQ], rq_col[NIWQ], rq_lds[NIWQ], rq_m32[NIWQ];
    uint64_t rq_m64[NIWQ];          // all ones for a V transfer: selects V's base and limit
#pragma unroll
    for (int m = 0; m < NIWQ; ++m) {
        const int i = min(wave + kNW * m, 2 * QR::NX - 1);
        const bool v = i >= QR::NX;
        const int x = v ? i - QR::NX : i, sl = 64 * x + lane;
        rq_off[m] = (uint32_t)(sl / QR::CPR) * growq;
        rq_col[m] = 12u * (uint32_t)(sl % QR::CPR);
        rq_lds[m] = __builtin_amdgcn_readfirstlane(
            lds_addr(lds + RAW0 + (v ? QR::KR * QR::RAWT : 0)) + (uint32_t)(1024 * x));
        rq_m32[m] = v ? ~0u : 0u;
        rq_m64[m] = v ? ~(uint64_t)0 : (uint64_t)0;
    }
    // the last row of the last tile (rows past it repeat it)
    const uint32_t lastq =
        nb > 0 ? (uint32_t)min((int64_t)kBN - 1, (int64_t)sk - 1 - (int64_t)(t0 + nb - 1) * kBN) : 0u;
    // iteration n's raw tiles: K(n+4) in page / tile slot sk4, V(n+2) in sv2; bases, row
    // limits and stage offsets, formed once and picked per transfer without a branch
    struct RawIt {
        uint64_t kb, vb;
        uint32_t kl, vl, ks, vs;
    };
    auto raw_it = [&](int n, int sk4, int sv2) INL {
        RawIt r;
        r.kb = (uint64_t)(kq + (int64_t)sk4 * kBN * growq);
        r.vb = (uint64_t)(vq + (int64_t)sv2 * kBN * growq);
        r.kl = (n + 4 >= nb - 1 ? lastq : (uint32_t)(kBN - 1)) * growq;
        r.vl = (n + 2 >= nb - 1 ? lastq : (uint32_t)(kBN - 1)) * growq;
        r.ks = (uint32_t)(((n + 4) & (QR::KR - 1)) * QR::RAWT);
        r.vs = (uint32_t)(((n + 2) % QR::VR) * QR::RAWT);
        return r;
    };
    auto dma_q4 = [&](const RawIt &r, int m) INL {
        const uint64_t base = r.kb ^ ((r.kb ^ r.vb) & rq_m64[m]);
        dma12c((const uint8_t *)base, rq_off[m], r.kl ^ ((r.kl ^ r.vl) & rq_m32[m]), rq_col[m],
               rq_lds[m], r.ks ^ ((r.ks ^ r.vs) & rq_m32[m]));
    };
    // mixed caches: this wave's m-th transfer, the TK of K(n+4) then the TV of V(n+2); the raw
    // tensor's NX wave-wide transfers are dealt to the waves (surplus ones repeat the last)
    // (the raw tensor's transfer mr moves column min(wave + 4 mr, NX - 1): fixed row offset,
    // column and LDS column, as for two raw tensors; the 16-bit tensor's go as dma_fast)
    constexpr int NRAW = ANYQ && !Q4 ? QR::NIW1 : 1;
    uint32_t mr_off[NRAW], mr_col[NRAW], mr_lds[NRAW];
#pragma unroll
    for (int mr = 0; mr < NRAW; ++mr) {
        const int sl = 64 * min(wave + kNW * mr, QR::NX - 1) + lane;
        mr_off[mr] = (uint32_t)(sl / QR::CPR) * growq;
        mr_col[mr] = 12u * (uint32_t)(sl % QR::CPR);
        mr_lds[mr] = __builtin_amdgcn_readfirstlane(
            lds_addr(lds + RAW0) + (uint32_t)(1024 * min(wave + kNW * mr, QR::NX - 1)));
    }
    auto dma_mixed = [&](int n, int m, int sk4, int sv2) INL {
        if (m < TK) {
            if constexpr (QK) {
                const int tl = n + 4;
                dma12c(kq + (int64_t)sk4 * kBN * growq, mr_off[m],
                       (tl >= nb - 1 ? lastq : (uint32_t)(kBN - 1)) * growq, mr_col[m], mr_lds[m],
                       (uint32_t)((tl & (QR::KR - 1)) * QR::RAWT));
            } else {
                dma_fast(n, m, sk4, sv2);
            }
        } else {
            const int mv = m - TK;
            if constexpr (QV) {
                const int tl = n + 2;
                dma12c(vq + (int64_t)sv2 * kBN * growq, mr_off[mv],
                       (tl >= nb - 1 ? lastq : (uint32_t)(kBN - 1)) * growq, mr_col[mv],
                       mr_lds[mv], (uint32_t)((tl % QR::VR) * QR::RAWT));
            } else {
                dma_fast(n, G::NDMA + mv, sk4, sv2);
            }
        }
    };
    // This thread's (key row, block) item of a tile: at D = 128 one K and one V item, wave w
    // taking the blocks of parity w & 1 (whether a block starts at byte 0 or 6 of its first
    // chunk is then wave-uniform); at D = 64 waves 0, 1 take K and waves 2, 3 V (block w & 1).
    const int dq_row = D == 128 ? 32 * (wave >> 1) + (lane & 31) : lane;
    const int dq_blk = D == 128 ? 2 * (lane >> 5) + (wave & 1) : (wave & 1);
    struct RawBlock {
        u32x4 A, Bq;
    };
    auto dq_load = [&](const uint8_t *raw) INL -> RawBlock {
        const uint8_t *sa = raw + 16 * (dq_row * QR::CPR + (3 * dq_blk) / 2);
        return RawBlock{*(const u32x4 *)sa, *(const u32x4 *)(sa + 16)};
    };
    // the item's f16 rows, in two halves: code dwords 2 h, 2 h + 1 into the chunks 4 blk + h
    // (low nibbles) and 4 blk + 2 + h (high nibbles), each half's stores issued before the next
    // half is unpacked (1.9 % faster at 2K x 16K than all unpacks first)
    auto dq_store = [&](const RawBlock &rb, uint8_t *dst, bool is_v) INL {
        const u32x4 &A = rb.A, &Bq = rb.Bq;
        uint32_t dbits, codes[4];
        if (wave & 1) {                            // odd block: 6 bytes into chunk A
            dbits = A[1] >> 16;
            codes[0] = A[2];
            codes[1] = Bq[0];
            codes[2] = Bq[1];
            codes[3] = Bq[2];
        } else {
            dbits = A[0] & 0xFFFFu;
            codes[0] = __builtin_amdgcn_alignbit(A[1], A[0], 16);
            codes[1] = __builtin_amdgcn_alignbit(A[2], A[1], 16);
            codes[2] = __builtin_amdgcn_alignbit(Bq[0], A[2], 16);
            codes[3] = __builtin_amdgcn_alignbit(Bq[1], Bq[0], 16);
        }
        const uint32_t d2 = dbits * 0x10001u;
        const int sw = is_v ? G::swv(dq_row) : G::swk(dq_row);
        uint8_t *rp = dst + dq_row * G::ROW;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            uint32_t lo[2][2], hi[2][2];
            q4_unpack_row(codes[2 * h2], d2, lo[0], hi[0]);
            q4_unpack_row(codes[2 * h2 + 1], d2, lo[1], hi[1]);
            *(u32x4 *)(rp + 16 * ((4 * dq_blk + h2) ^ sw)) = (u32x4){lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
            *(u32x4 *)(rp + 16 * ((4 * dq_blk + 2 + h2) ^ sw)) = (u32x4){hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
        }
    };
    auto dequant_k = [&](int tl) INL {
        if (D == 128 || wave < 2)
            dq_store(dq_load(rawk(tl)), kstage(tl), false);
    };
    auto dequant_v = [&](int tl) INL {
        if (D == 128 || wave >= 2)
            dq_store(dq_load(rawv(tl)), vstage(tl), true);
    };
    // K tile tk and V tile tv together: both raw reads are issued before either item's stores
    // (the compiler cannot move a read of the raw stages past a store into the f16 rings)
    auto dequant_kv = [&](int tk, int tv) INL {
        if constexpr (D == 128) {
            const RawBlock rk = dq_load(rawk(tk)), rv = dq_load(rawv(tv));
            dq_store(rk, kstage(tk), false);
            dq_store(rv, vstage(tv), true);
        } else if (wave < 2) {
            dq_store(dq_load(rawk(tk)), kstage(tk), false);
        } else {
            dq_store(dq_load(rawv(tv)), vstage(tv), true);
        }
    };

    // ---- fragment addressing -----------------------------------------------------------------
    // K fragment f (hf = f / NST, st = f % NST): row krow = hf*32 + perm(col), chunk 2*st + half;
    // byte offset krow*ROW + 16*((2*st + half) ^ swk(krow)) = (krow*ROW | X) ^ 32*st
    const int krow0 = k_row_perm16(col);
    const uint32_t kfx = (uint32_t)(krow0 * G::ROW) | (uint32_t)(16 * (half ^ G::swk(krow0)));
    auto kread = [&](const uint8_t *ks, int f) INL -> u32x4 {
        const int hf = f / NST, st = f % NST;
        return *(const u32x4 *)(ks + (kfx ^ (uint32_t)(32 * st)) + hf * 32 * G::ROW);
    };
    // V^T fragment f (t4 = f / NDT, dt = f % NDT) via transpose reads: group g = lane/16,
    // position jl = lane%16 as a source lane reads
    // V[16*t4 + 8*(g/2) + 4*sec + jl/4][32*dt + 16*(g%2) + 4*(jl%4) .. +3]
    const int g = lane >> 4, jl = lane & 15;
    const int vr0 = 8 * (g >> 1) + (jl >> 2);                 // row within a 16-key group
    const int vchunk = 2 * (g & 1) + ((jl & 3) >> 1);         // chunk within a 32-column block
    const uint32_t vfx = (uint32_t)(vr0 * G::ROW) +
                         (uint32_t)(16 * (vchunk ^ G::swv(vr0)) + 8 * (jl & 1));
    // for dt: chunk 4*dt + vchunk, swizzled: (4*dt) ^ swv only touches bits the dt term owns
    auto vread = [&](const uint8_t *vs, int f) INL -> u32x4 {
        const int t4 = f / NDT, dt = f % NDT;
        const uint32_t o = (vfx ^ (uint32_t)(64 * dt)) + (uint32_t)(16 * t4 * G::ROW);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vs + o));
        const s16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vs + o + 4 * G::ROW));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return (u32x4){l2[0], l2[1], h2[0], h2[1]};
    };

    // ---- softmax of block j over the scores s (S^T registers of tile n) ------------------------
    u32x4 pf[2][4];
    float m8[2][8], mx[2], m2[2];
    bool need[2];
    float pv2[2][16][2];                           // P values between an E unit and its C unit
    // tiles n >= nmask[j] hold a key that some row of block j cannot see: for them
    // (t0 + n) * kBN + kBN - 1 > klim_min[j], i.e. n >= floor((klim_min[j] + 1) / kBN) - t0
    int nmask[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t x = klim_min[j] + 1;
        const int64_t fl = x >= 0 ? x / kBN : -((-x + kBN - 1) / kBN);
        nmask[j] = (int)max((int64_t)0, min((int64_t)nb, fl - t0));
    }
    auto mask = [&](int j, f32x16 *s, int n) INL {
        const int k0 = (t0 + n) * kBN;
        if (n >= nmask[j]) {
            const int lim = (int)max(min(klim[j] - k0, (int64_t)kBN), (int64_t)-1) - 8 * half;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (hf * 32 + 16 * (i / 8) + (i % 8) > lim)
                        s[hf][i] = -INFINITY;
        }
    };
    // softmax unit number ic of the schedule (see make_schedule), of block x.j
    auto run_unit = [&](auto ic, f32x16 *s0, f32x16 *s1) INL {
        constexpr Unit x = PL::sc.unit[decltype(ic)::value];
        constexpr int j = x.j;
        f32x16 *s = j == 0 ? s0 : s1;
        if constexpr (x.kind == UM) {
            constexpr int u = x.idx;
            m8[j][u] = vmax(vmax3(s[0][2 * u], s[0][2 * u + 1], s[1][2 * u]), s[1][2 * u + 1]);
            pin(m8[j][u]);
        } else if constexpr (x.kind == UT1) {
            m8[j][0] = vmax3(m8[j][0], m8[j][1], m8[j][2]);
            m8[j][3] = vmax3(m8[j][3], m8[j][4], m8[j][5]);
            m8[j][6] = vmax(m8[j][6], m8[j][7]);
            pin(m8[j][0]);
            pin(m8[j][3]);
            pin(m8[j][6]);
        } else if constexpr (x.kind == UT2) {
            m8[j][0] = vmax3(m8[j][0], m8[j][3], m8[j][6]);
            pin(m8[j][0]);
        } else if constexpr (x.kind == UP) {
            mx[j] = pair_max(m8[j][0]);
            pin(mx[j]);
        } else if constexpr (x.kind == UF1) {
            m2[j] = mx[j] * a.c;
            need[j] = m2[j] > frame[j] + kRescaleMarginLog2;
            pin(m2[j]);
        } else if constexpr (x.kind == UF2) {
            alpha[j] = need[j] ? exp2_fast(frame[j] - m2[j]) : 1.0f;
            frame[j] = need[j] ? m2[j] : frame[j];
            fr[j] = (frame[j] == -INFINITY) ? 0.0f : frame[j];
            lsum[j] *= alpha[j];
            rescale[j] = __any(need[j]);
            if constexpr (STATS) {
                nmove[j] += need[j] ? 1 : 0;
                nresc[j] += rescale[j] ? 1 : 0;
            }
            pin(fr[j]);
        } else if constexpr (x.kind == UE) {
            constexpr int t4 = x.idx >> 2, e = x.idx & 3, i = 8 * (t4 & 1) + 2 * e;
            pv2[j][x.idx][0] = exp2_fast(__builtin_fmaf(s[t4 >> 1][i], a.c, -fr[j]));
            pv2[j][x.idx][1] = exp2_fast(__builtin_fmaf(s[t4 >> 1][i + 1], a.c, -fr[j]));
            pin(pv2[j][x.idx][0]);
            pin(pv2[j][x.idx][1]);
        } else {
            constexpr int t4 = x.idx >> 2, e = x.idx & 3;
            uint32_t pk = pack2<BF>(pv2[j][x.idx][0], pv2[j][x.idx][1]);
            pin(pk);
            pf[j][t4][e] = pk;
            lsum[j] = sum2<BF>(pk, lsum[j]);
        }
    };
    auto apply_rescale = [&](int j) INL {
        if (rescale[j]) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                acc[j][dt] *= alpha[j];
        }
    };

    // ---- MFMA slots ----------------------------------------------------------------------------
    // P.V slot i: V^T fragment i/2 times P of block i%2; score slot i: K fragment i/2 times Q
    // of block i%2 (fragments in hf-major order, so block 0's hf = 0 chain finishes first)
    auto pv_slot = [&](int i, const u32x4 &vf) INL {
        const int f = i >> 1, j = i & 1, t4 = f / NDT, dt = f % NDT;
        acc[j][dt] = mfma32<BF>(vf, pf[j][t4], acc[j][dt]);
    };
    auto s_slot = [&](int i, const u32x4 &kf, f32x16 *s0, f32x16 *s1) INL {
        const int f = i >> 1, j = i & 1, hf = f / NST, st = f % NST;
        f32x16 *s = j == 0 ? s0 : s1;
        if (st == 0)
            smfma_first<BF>(s[hf], kf, qf[j][st]);
        else
            smfma_acc<BF>(s[hf], kf, qf[j][st]);
    };
    // Fragment reads run kRead fragments ahead of their MFMAs through a ring of kRead + 1
    // registers; sched_barrier fences keep the compiler from hoisting every read at once.
    // Timed on an MI355X (same outputs): 4 ahead at D = 128 0.3-0.6 % faster than 3 on the
    // f16, q4_0 and paged prefills (bf16 and mixed unchanged), 3 at D = 64 1.5 % faster than 4.
    constexpr int kRead = D == 128 ? 4 : 3;
    auto scores_all = [&](const uint8_t *ks, f32x16 *s0, f32x16 *s1) INL {
        u32x4 fb[kRead + 1];
        static_for<0, kRead>([&](auto fc) { fb[fc.value] = kread(ks, fc.value); });
        static_for<0, 2 * NST>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f + kRead < 2 * NST)
                fb[(f + kRead) % (kRead + 1)] = kread(ks, f + kRead);
            s_slot(2 * f, fb[f % (kRead + 1)], s0, s1);
            s_slot(2 * f + 1, fb[f % (kRead + 1)], s0, s1);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto pv_all = [&](const uint8_t *vs) INL {
        u32x4 fb[kRead + 1];
        static_for<0, kRead>([&](auto fc) { fb[fc.value] = vread(vs, fc.value); });
        static_for<0, 4 * NDT>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f + kRead < 4 * NDT)
                fb[(f + kRead) % (kRead + 1)] = vread(vs, f + kRead);
            pv_slot(2 * f, fb[f % (kRead + 1)]);
            pv_slot(2 * f + 1, fb[f % (kRead + 1)]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // One tile: a fixed slot sequence, fragment reads kRead fragments ahead, softmax units
    // and DMA transfers at planned slots; sched_barrier fences keep the order. Every tile runs
    // the same sequence: where a wave has nothing to do the work is harmless (P of tile -1 is
    // zero against a zeroed V stage, scores of a tile past the last are never used, keys a row
    // cannot see are masked to -inf and give P = 0).
    auto tile = [&](int n, f32x16 *s0, f32x16 *s1c, f32x16 *s1n) INL {
        const uint8_t *vs = vstage(n - 1), *ks = kstage(n + 1);
        const int sk4 = slot(n + LK), sv2 = slot(n + LV);   // where this iteration's DMA reads
        RawIt rit{};
        if constexpr (Q4)
            rit = raw_it(n, sk4, sv2);                   // (LK = 4, LV = 2 here)
        u32x4 fb[kRead + 1];
        // Both caches q4_0 at D = 128: K(n+2) and V(n) are dequantized inside half 2, the raw
        // blocks read in slot NM + 4 and K's and V's f16 rows written in slots NM + 14 and
        // NM + 26 (into the stages of K(n) and V(n-2), read in iteration n-1; the raw tiles
        // landed before the barrier). Timed on an MI355X against the end of the tile and four
        // other placements: 1.8-1.9 % faster at 2K x 16K, 3-4 % for 256 queries; half 1 was
        // slower, and with one q4_0 cache the end of the tile stays (0.6 % faster there).
        constexpr bool DQS = Q4 && D == 128;
        constexpr int DQL = NM + 4, DQK = NM + 14, DQV = NM + 26;
        RawBlock dqk{}, dqv{};
        auto dq_at = [&](auto sl_) INL {
            constexpr int sl = decltype(sl_)::value;
            if constexpr (DQS) {
                if constexpr (sl == DQL) {
                    if constexpr (QK)
                        dqk = dq_load(rawk(n + 2));
                    if constexpr (QV)
                        dqv = dq_load(rawv(n));
                }
                if constexpr (QK && sl == DQK)
                    dq_store(dqk, kstage(n + 2), false);
                if constexpr (QV && sl == DQV)
                    dq_store(dqv, vstage(n), true);
            }
        };
        auto units = [&](auto sc_) INL {          // the softmax units of slot sc_
            constexpr int sl = decltype(sc_)::value;
            static_for<PL::sc.first[sl], PL::sc.first[sl + 1]>([&](auto ic) INL {
                run_unit(ic, s0, s1c);
            });
        };
        // half 1: P.V of tile n-1 for both blocks
        static_for<0, kRead>([&](auto fc) INL { fb[fc.value] = vread(vs, fc.value); });
        static_for<0, NM>([&](auto ic) INL {
            constexpr int i = decltype(ic)::value, f = i >> 1;
            if constexpr ((i & 1) == 0 && f + kRead < 4 * NDT)
                fb[(f + kRead) % (kRead + 1)] = vread(vs, f + kRead);
            pv_slot(i, fb[f % (kRead + 1)]);
            if constexpr (i == 0) {
                // the first VALU reads of this tile's scores wait here, while the first P.V
                // MFMA (which does not read them) runs
                __builtin_amdgcn_sched_barrier(0);
                smfma_drain(s0[0], s0[1], s1c[0], s1c[1]);
                mask(0, s0, n);
                mask(1, s1c, n);
            }
            units(ic);
            dq_at(ic);
            if constexpr (FAST16 && kDmaMode == 2 && (i & 3) == 1 && (i >> 2) < G::NDMA)
                dma_fast(n, i >> 2, sk4, sv2);        // K(n+LK)
            __builtin_amdgcn_sched_barrier(0);
        });
        // half 2: scores of tile n+1 for both blocks
        static_for<0, kRead>([&](auto fc) INL { fb[fc.value] = kread(ks, fc.value); });
        static_for<0, NM>([&](auto ic) INL {
            constexpr int i = decltype(ic)::value, f = i >> 1;
            if constexpr ((i & 1) == 0 && f + kRead < 2 * NST)
                fb[(f + kRead) % (kRead + 1)] = kread(ks, f + kRead);
            s_slot(i, fb[f % (kRead + 1)], s0, s1n);
            units(std::integral_constant<int, NM + i>{});
            dq_at(std::integral_constant<int, NM + i>{});
            if constexpr (Q4) {
                if constexpr ((i & 3) == 1 && (i >> 2) < QR::NIW)
                    dma_q4(rit, i >> 2);
            } else if constexpr (ANYQ) {
                if constexpr ((i & 3) == 1 && (i >> 2) < TI)
                    dma_mixed(n, i >> 2, sk4, sv2);
            } else if constexpr ((i & 3) == 1 && (i >> 2) < 2 * G::NDMA) {
                constexpr int m = i >> 2;
                if constexpr (kDmaMode == 0)
                    dma_fast(n, m, sk4, sv2);
                else if constexpr (kDmaMode == 2 && m < G::NDMA)
                    dma_fast(n, G::NDMA + m, sk4, sv2);   // V(n+LV)
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (FAST16)
            dma_advance(n);
        static_for<PL::sc.first[2 * NM], kNU>([&](auto ic) INL { run_unit(ic, s0, s1c); });
        // O of both blocks rescaled (rarely) between the last P.V of the old frame (half 1) and
        // the first of the new (half 1 of the next tile)
        apply_rescale(0);
        apply_rescale(1);
        if constexpr (ANYQ && !DQS) {
            // K(n+2) and V(n) into the stages of K(n) and V(n-2), read in iteration n-1 (at the
            // end of the tile, where the last score MFMAs are still executing)
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (Q4)
                dequant_kv(n + 2, n);
            else if constexpr (QK)
                dequant_k(n + 2);
            else
                dequant_v(n);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- pipeline --------------------------------------------------------------------------------
    // Iteration n reads K(n+1) and V(n-1) and refills the stages of K(n) and V(n-2), which the
    // barrier shows every wave is done with, with K(n+4) and V(n+2). Before barrier n the
    // transfers issued in iterations n-1 and n-2 (2 tiles each) may still be in flight,
    // nothing older.
    auto wait_tiles = [&](int pend_tiles) INL {
        if (pend_tiles >= 4)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4 * G::NDMA));
        else if (pend_tiles >= 2)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * G::NDMA));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        asm volatile("s_barrier" ::: "memory");
    };
    // prologue: K(0..3), V(0..1) (q4_0: raw, the transfers dealt round-robin to the waves)
    if (nb > 0) {
        if constexpr (QK) {
#pragma unroll
            for (int tl = 0; tl < 4; ++tl)
#pragma unroll
                for (int x = 0; x < QR::NX; ++x)
                    if (x % kNW == wave)
                        dma_raw(false, tl, slot(tl), x);
        } else {
#pragma unroll
            for (int tl = 0; tl < LK; ++tl)
#pragma unroll
                for (int i = 0; i < G::NDMA; ++i)
                    dma_one(false, tl, tl, slot(tl), i);
        }
        if constexpr (QV) {
#pragma unroll
            for (int tl = 0; tl < 2; ++tl)
#pragma unroll
                for (int x = 0; x < QR::NX; ++x)
                    if (x % kNW == wave)
                        dma_raw(true, tl, slot(tl), x);
        } else {
#pragma unroll
            for (int tl = 0; tl < LV; ++tl)
#pragma unroll
                for (int i = 0; i < G::NDMA; ++i)
                    dma_one(true, FSK + tl, tl, slot(tl), i);
        }
    }

    // The V stage of tile -1 holds zeros, so that P.V of tile -1 adds nothing (P is zero too);
    // tile FSV-1 is written into it only after barrier 1 (by a transfer or the dequantization)
    {
        uint8_t *z = vstage(-1);
        for (int o = t * 16; o < G::TILE; o += kNT * 16)
            *(u32x4 *)(z + o) = (u32x4){0u, 0u, 0u, 0u};
        for (int i = 0; i < 4; ++i)
            pf[0][i] = pf[1][i] = (u32x4){0u, 0u, 0u, 0u};
    }
    f32x16 s0[2], s1a[2], s1b[2];
    auto iteration = [&](int n, f32x16 *s1c, f32x16 *s1n) INL {
        if constexpr (ANYQ) {
            // raw K(n+2) and V(n) landed: only iteration n-1's transfers may be in flight
            // (with one f16 tensor its tiles landed earlier still)
            if (n >= 1)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(TI));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
            asm volatile("s_barrier" ::: "memory");
        } else if constexpr (PAIR) {
            // even n: K(n+1), K(n+2), V(n-1), V(n) resident (issued by iteration n-5 or the
            // prologue), so iterations n-4 .. n-1 may have transfers in flight; odd n relies
            // on the barrier of n-1
            if ((n & 1) == 0) {
                if (n >= 4)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4 * 2 * G::NDMA));
                else if (n >= 2)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * 2 * G::NDMA));
                else
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
                asm volatile("s_barrier" ::: "memory");
            }
        } else {
            // iterations n-1 and n-2 may have transfers in flight (none yet at n = 0, 1: the
            // wait before the loop drained the prologue's)
            wait_tiles(4);
        }
        tile(n, s0, s1c, s1n);
    };
    if (nb > 0) {
        wait_tiles(0);           // K(0) resident; also orders the zero fill before its reads
        if constexpr (QK) {
            dequant_k(0);
            dequant_k(1);
            wait_tiles(0);
        }
        scores_all(kstage(0), s0, s1a);
    }
    for (int n = 0; n < nb; n += 2) {
        iteration(n, s1a, s1b);
        if (n + 1 < nb)
            iteration(n + 1, s1b, s1a);
    }
    // the last tile's P.V: its V may have been in flight at the last barrier
    wait_tiles(0);
    if (nb >= 1)
        pv_all(vstage(nb - 1));

    // ---- epilogue ----------------------------------------------------------------------------
    if constexpr (SPLIT) {
        if (p.parts > 0) {
            // key split: this run's rows (unnormalised O, frame, sum) go to the workspace as
            // contiguous runs through LDS (the tile rings, free after the last tile), for the
            // merge kernel that follows
            static_assert(LDSB >= kNW * 32 * kPartRow * 4, "staging fits the tile rings");
            constexpr int RUN = 32 * kPartRow;
            float *mine = p.part + (((int64_t)unit_id * p.parts + run_id) * kNW + wave) *
                                       (int64_t)(2 * RUN);
            float *stg = (float *)lds + wave * RUN;
            float *row = stg + col * kPartRow;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float ltot = pair_sum(lsum[j]);
                __syncthreads();
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        *(f32x4 *)(row + 32 * dt + 8 * ii + 4 * half) =
                            f32x4{acc[j][dt][4 * ii + 0], acc[j][dt][4 * ii + 1],
                                  acc[j][dt][4 * ii + 2], acc[j][dt][4 * ii + 3]};
                if (half == 0)
                    *(f32x2 *)(row + D) = f32x2{frame[j], ltot};
                __syncthreads();
#pragma unroll
                for (int e = 4 * lane; e < RUN; e += 256)
                    *(f32x4 *)(mine + j * RUN + e) = *(const f32x4 *)(stg + e);
            }
            return;
        }
        if (split_unit) {
            // This part's rows (unnormalised O, frame, sum) go to the workspace; the later of
            // the unit's two parts merges them: F = max f, O = sum 2^(f - F) O_f / sum 2^(f - F)
            // l_f. Rows pass through LDS (the tile rings, free once every wave is past its
            // last tile) so that the workspace is written and read in contiguous runs, one
            // 32-row block of a wave (32 x kPartRow floats) at a time.
            static_assert(LDSB >= kNW * 32 * kPartRow * 4, "staging fits the tile rings");
            constexpr int RUN = 32 * kPartRow;              // floats of one wave's block
            const int64_t su = (((int64_t)b * a.Hkv + kvh) * p.n_hchunk + hc) *
                                   (p.n_qblk - p.q_split) + (qblk - p.q_split);
            float *mine = p.part + ((su * 2 + part) * kNW + wave) * (int64_t)(2 * RUN);
            const float *other = p.part + ((su * 2 + (1 - part)) * kNW + wave) * (int64_t)(2 * RUN);
            float *stg = (float *)lds + wave * RUN;
            float *row = stg + col * kPartRow;
            float ltot[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                ltot[j] = pair_sum(lsum[j]);
                __syncthreads();
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        *(f32x4 *)(row + 32 * dt + 8 * ii + 4 * half) =
                            f32x4{acc[j][dt][4 * ii + 0], acc[j][dt][4 * ii + 1],
                                  acc[j][dt][4 * ii + 2], acc[j][dt][4 * ii + 3]};
                if (half == 0)
                    *(f32x2 *)(row + D) = f32x2{frame[j], ltot[j]};
                __syncthreads();
#pragma unroll
                for (int e = 2 * lane; e < RUN; e += 128)
                    store_through2(mine + j * RUN + e, stg[e], stg[e + 1]);
            }
            if (!arrive_last(p.cnt + su, 2u, &arrived))
                return;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x2 in[(RUN + 127) / 128];
#pragma unroll
                for (int u = 0; u < (RUN + 127) / 128; ++u)
                    in[u] = load_through2(other + j * RUN + min(2 * lane + 128 * u, RUN - 2));
                __syncthreads();
#pragma unroll
                for (int u = 0; u < (RUN + 127) / 128; ++u)
                    if (2 * lane + 128 * u < RUN)
                        *(f32x2 *)(stg + 2 * lane + 128 * u) = in[u];
                __syncthreads();
                const f32x2 fl = *(const f32x2 *)(row + D);
                const float F = fmaxf(frame[j], fl[0]);
                const float wm = F == -INFINITY ? 0.0f : exp2_fast(frame[j] - F);
                const float wo = F == -INFINITY ? 0.0f : exp2_fast(fl[0] - F);
                // part 0's terms first, whichever part merges, so the rows do not depend on
                // which of the two finished last: w0 y0 + w1 y1 as one fma over one product
                const bool p0 = part == 0;
                const float w0 = p0 ? wm : wo, w1 = p0 ? wo : wm;
                auto mix = [&](float ym, float yo) INL {
                    return __builtin_fmaf(w0, p0 ? ym : yo, w1 * (p0 ? yo : ym));
                };
                const float L = mix(ltot[j], fl[1]);
                if (!wave_on || qi[j] >= sq)
                    continue;
                const float inv = L > 0.0f ? 1.0f / L : 0.0f;
                uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi[j]) * a.Hq + h) * D;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const f32x4 x = *(const f32x4 *)(row + 32 * dt + 8 * ii + 4 * half);
                        const f32x16 &c = acc[j][dt];
                        u32x2 w;
                        w[0] = pack2<BF>(mix(c[4 * ii + 0], x[0]) * inv,
                                         mix(c[4 * ii + 1], x[1]) * inv);
                        w[1] = pack2<BF>(mix(c[4 * ii + 2], x[2]) * inv,
                                         mix(c[4 * ii + 3], x[3]) * inv);
                        *(u32x2 *)(op + 32 * dt + 8 * ii + 4 * half) = w;
                    }
            }
            return;
        }
    }
    // The wave's 64 normalised rows go out through LDS: written from the accumulators (lane =
    // row, 8 bytes of 4 d values per write) into the wave's own 64 x 2D-byte region of the
    // tile rings, 16-byte chunk c of row r at slot c ^ (r % CPR), then read back and stored
    // as whole rows, 16 bytes a lane. Straight from the accumulators every store instruction
    // would touch 32 rows. Every transfer has landed (wait_tiles above); the barrier waits
    // for the other waves' last P.V reads (with a raw q4_0 K the V ring lies in the region).
    static_assert(LDSB >= kNW * 64 * G::ROW, "the rows fit the tile rings");
    uint8_t *orow = lds + wave * 64 * G::ROW;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float ltot = pair_sum(lsum[j]);
        const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
        if constexpr (STATS) {
            if (wave_on && qi[j] < sq && half == 0)
                *(int2 *)(p.stats + 2 * (((int64_t)b * a.Sq + qi[j]) * a.Hq + h)) =
                    make_int2(nmove[j], nresc[j]);
        }
        const int r = 32 * j + col;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                u32x2 w;
                w[0] = pack2<BF>(acc[j][dt][4 * ii + 0] * inv, acc[j][dt][4 * ii + 1] * inv);
                w[1] = pack2<BF>(acc[j][dt][4 * ii + 2] * inv, acc[j][dt][4 * ii + 3] * inv);
                const int c = 4 * dt + ii;
                *(u32x2 *)(orow + r * G::ROW + ((c ^ (r % G::CPR)) * 16) + 8 * half) = w;
            }
    }
    // the wave reads back its own region: its LDS writes complete first, and the clobber keeps
    // the compiler from moving the reads above them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (wave_on) {
        constexpr int RPI = 64 / G::CPR;                 // rows per store instruction
#pragma unroll
        for (int s_ = 0; s_ < 64 / RPI; ++s_) {
            const int r = s_ * RPI + lane / G::CPR, c = lane % G::CPR;
            const u32x4 x = *(const u32x4 *)(orow + r * G::ROW + ((c ^ (r % G::CPR)) * 16));
            if (q0 + r < sq)
                *(u32x4 *)((uint16_t *)a.o + (((int64_t)b * a.Sq + q0 + r) * a.Hq + h) * D +
                           8 * c) = x;
        }
    }
    };  // run

    run(qblk0, 0);
    if constexpr (SPLIT) {
        // a light unit then runs the tiles past the cap of its mirror unit n - 1 - q, whose
        // tile count rises as this one's falls
        const int partner = p.n_qblk - 1 - qblk0;
        if (qblk0 < p.q_split && partner >= p.q_split) {
            __syncthreads();   // every wave is done with the LDS of the first unit
            run(partner, 1);
        }
    }
}

// Key split: combine the runs of each unit's rows. One workgroup per (unit, wave): thread t
// takes row t / 4 of the wave's 64 and a quarter of its D outputs; with the runs' frames f_r and
// sums l_r, F = max f_r and O = sum 2^(f_r - F) O_r / sum 2^(f_r - F) l_r (a run that saw no key
// has f_r = -inf and weight 0; a row no run saw gets O = 0).
template <int D, bool BF>
__global__ __launch_bounds__(256) void prefill_parts_merge_kernel(Prefill16Params p)
{
    constexpr int RUN = 32 * kPartRow, QD = D / 4;
    const AttnArgs &a = p.a;
    const int wave = blockIdx.x % kNW, unit_id = blockIdx.x / kNW;
    int rest = unit_id;
    const int qbl = rest % p.n_qblk;
    rest /= p.n_qblk;
    const int hc = rest % p.n_hchunk;
    rest /= p.n_hchunk;
    const int kvh = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int qblk = a.causal ? p.n_qblk - 1 - qbl : qbl;
    const int hs = wave % p.hpw, qs = wave / p.hpw;
    const int hl = hc * p.hpw + hs;
    const int q0 = qblk * kQW * p.qsub + qs * kQW;
    if (wave >= p.hpw * p.qsub || hl >= a.G || q0 >= a.Sq)
        return;                                      // a wave slot with no rows
    const int h = kvh * a.G + hl;
    const int r = threadIdx.x >> 2, qd = threadIdx.x & 3;
    const int qi = q0 + r;                           // row r: block r / 32, column r % 32
    if (qi >= a.Sq)
        return;
    const float *base = p.part + (int64_t)unit_id * p.parts * kNW * 2 * RUN +
                        (int64_t)wave * 2 * RUN + (r >> 5) * RUN + (r & 31) * kPartRow;
    const int64_t rstride = (int64_t)kNW * 2 * RUN;  // between runs of the unit
    float F = -INFINITY;
    for (int k = 0; k < p.parts; ++k)
        F = fmaxf(F, base[k * rstride + D]);
    float L = 0.0f;
    f32x4 o[QD / 4];
#pragma unroll
    for (int e = 0; e < QD / 4; ++e)
        o[e] = (f32x4){};
    if (F != -INFINITY) {
        for (int k = 0; k < p.parts; ++k) {
            const float *src = base + k * rstride;
            const float w = exp2_fast(src[D] - F);
            L += w * src[D + 1];
#pragma unroll
            for (int e = 0; e < QD / 4; ++e)
                o[e] += w * *(const f32x4 *)(src + qd * QD + 4 * e);
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t *op = (uint16_t *)a.o + (((int64_t)b * a.Sq + qi) * a.Hq + h) * D + qd * QD;
#pragma unroll
    for (int e = 0; e < QD / 4; ++e)
        *(u32x2 *)(op + 4 * e) = (u32x2){pack2<BF>(o[e][0] * inv, o[e][1] * inv),
                                         pack2<BF>(o[e][2] * inv, o[e][3] * inv)};
}

template <int D, int KT, int VT>
hipError_t launch16(const Prefill16Params &p, int64_t n_wg, hipStream_t stream)
{
    // the split instances: 16-bit caches at both head dims; a q4_0 tensor at D = 128 only (at
    // D = 64 its kernel's LDS is smaller than the split's staging)
    if constexpr (D == 128 || (KT != KV_Q4_0 && VT != KV_Q4_0)) {
        if (p.cnt) {
            hipLaunchKernelGGL((prefill16_kernel<D, KT, VT, false, true>),
                               dim3((unsigned)p.n_main), dim3(kNT), 0, stream, p);
            if (p.parts > 0) {
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess)
                    return e;
                hipLaunchKernelGGL((prefill_parts_merge_kernel<D, KT == KV_BF16>),
                                   dim3((unsigned)(p.n_main / p.parts * kNW)), dim3(256), 0,
                                   stream, p);
            }
            return hipGetLastError();
        }
    }
    // the counter instances: D = 128, one cache type for K and V
    if constexpr (D == 128 && KT == VT) {
        if (p.stats) {
            hipLaunchKernelGGL((prefill16_kernel<D, KT, VT, false, false, true>),
                               dim3((unsigned)n_wg), dim3(kNT), 0, stream, p);
            return hipGetLastError();
        }
    }
    if (p.stats)
        return hipErrorInvalidValue;
    if (p.block_table)
        hipLaunchKernelGGL((prefill16_kernel<D, KT, VT, true>), dim3((unsigned)n_wg), dim3(kNT),
                           0, stream, p);
    else
        hipLaunchKernelGGL((prefill16_kernel<D, KT, VT, false>), dim3((unsigned)n_wg), dim3(kNT),
                           0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch16_kv(const Prefill16Params &p, int64_t n_wg, hipStream_t stream)
{
    switch (p.a.kv) {
    case KV_BF16:
        return launch16<D, KV_BF16, KV_BF16>(p, n_wg, stream);
    case KV_Q4_0:
        return launch16<D, KV_Q4_0, KV_Q4_0>(p, n_wg, stream);
    case KV_F16_Q4_0:
        return launch16<D, KV_F16, KV_Q4_0>(p, n_wg, stream);
    case KV_Q4_0_F16:
        return launch16<D, KV_Q4_0, KV_F16>(p, n_wg, stream);
    default:
        return launch16<D, KV_F16, KV_F16>(p, n_wg, stream);
    }
}

}  // namespace

// Balanced causal split: the units' tile counts grow with the query block, linearly where
// every row sees the keys up to its own position. Query blocks q and n - 1 - q together hold
// about twice the average, so the heavier of the two (q >= q_split, q_split >= n / 2) runs
// its first `cap` tiles and the lighter one runs the rest after its own, in the same
// workgroup: cap = the average tiles per unit plus kSplitBias, which leaves the light
// workgroup the time to restart (load the second unit's Q and first tiles) and merge. Timed
// on an MI355X at 2K, 8K and 16K keys, biases 0-6: 3 was best (4 close, 0 and 6 worst).
constexpr int kSplitBias = 3;

// Key split: when the units are at most half the CUs (a short chunk of queries against many
// keys, where each workgroup would run its unit's tiles alone while most CUs idle), every
// unit's tiles are cut into `parts` runs of at least kMinRunTiles tiles, as many as fill the
// kCUs CUs in one round (parts = kCUs / units), merged by a second kernel. Timed on an MI355X at
// 8-128 units and 2K-16K keys against runs sized for two or four rounds (512 or 1024
// workgroups): one round was fastest at every shape (e.g. 1024 queries x 16K keys: 267 us
// against 278 and 307; 64 queries: 78 against 130). With more units than that and at most
// kCUs, pairing. With more than kCUs units the workgroups run in several rounds, and the
// hardware's dispatch of the later rounds onto the CUs that free up (heaviest units first)
// already evens the load: nothing is paired. Timed on an MI355X against pairing there: 4096
// queries x 4096 keys 143 against 163 us, 3072 x 3072 94 against 120, two sequences of
// 2048 x 2048 83 against 105, 8192 x 8192 508 against 544.
constexpr int64_t kCUs = 256;          // compute units of the gfx950 part (MI355X)
constexpr int64_t kMinRunTiles = 4;
constexpr int64_t kMaxParts = 64;

// Dequantize first: the fused kernel dequantizes a q4_0 tile in every workgroup that reads it,
// once per query block and head chunk of its KV head; widening the cache to f16 once costs a
// pass over it. Timed at 16K keys, GQA 32/8 (fa_prefill_split both ways, same GPU): 64-256
// queries (1-4 blocks) fused faster (118-135 us against 138-161), 512 (8) even, 1024 (16) and
// more the dequantized copy faster. Output bits are the same either way (one unpack routine).
constexpr int64_t kDequantFirstBlocks = 16;

PrefillSplit prefill_split_plan(const AttnArgs &a0)
{
    PrefillSplit sp{};
    if ((int64_t)a0.B * a0.Sq == 0)
        return sp;
    const PrefillGrid g = prefill16_grid(a0);
    AttnArgs a = a0;
    const bool qk = a0.kv == KV_Q4_0 || a0.kv == KV_Q4_0_F16;
    const bool qv = a0.kv == KV_Q4_0 || a0.kv == KV_F16_Q4_0;
    const int64_t n_blocks = (int64_t)a0.B * a0.Sk * a0.Hkv * (a0.D / 32);
    if ((qk || qv) && (int64_t)g.n_qblk * g.n_hchunk >= kDequantFirstBlocks &&
        n_blocks / 256 < INT32_MAX) {                             // the dequant grid fits

        sp.deq = (qk ? 1 : 0) | (qv ? 2 : 0);
        sp.deq_bytes = (size_t)a0.B * a0.Sk * a0.Hkv * a0.D * 2;
        a.kv = KV_F16;
    }
    // the workspace: arrival counters and partial rows, then any f16 copies (after the counter
    // bytes even when nothing is split, so a later call that shares the workspace finds its
    // counters at zero)
    auto finish = [&](PrefillSplit s) {
        if (s.deq) {
            s.deq_off = (std::max(s.workspace_bytes, kSplitCounterBytes) + 255) & ~(size_t)255;
            s.workspace_bytes = s.deq_off + (size_t)((s.deq & 1) + (s.deq >> 1)) * s.deq_bytes;
        }
        return s;
    };
    const bool q4 = a.kv == KV_Q4_0 || a.kv == KV_F16_Q4_0 || a.kv == KV_Q4_0_F16;
    if (q4 && a.D != 128)
        return finish(sp);
    const int bmq = kQW * g.qsub;
    auto tiles = [&](int qblk) -> int64_t {
        const int64_t qlast = std::min((int64_t)qblk * bmq + bmq, (int64_t)a.Sq) - 1;
        int64_t kend = a.causal ? std::min((int64_t)a.Sk, qlast + a.offset + 1) : (int64_t)a.Sk;
        kend = kend < 0 ? 0 : kend;
        return (kend + kBN - 1) / kBN;
    };
    const int64_t per = (int64_t)g.n_hchunk * a.Hkv * a.B;       // units per query block
    const int64_t n_units = (int64_t)g.n_qblk * per;
    const int64_t t_max = tiles(a.causal ? g.n_qblk - 1 : 0);
    const size_t unit_part_bytes = (size_t)kNW * kQW * kPartRow * 4;   // one run of one unit
    {
        const int64_t parts = std::min(kCUs / n_units, std::min(kMaxParts, t_max / kMinRunTiles));
        if (parts >= 2) {
            sp.parts = (int)parts;
            sp.q_split = g.n_qblk;                               // no unit is paired
            sp.n_main = n_units * parts;
            sp.n_tail = n_units;
            sp.workspace_bytes = kSplitCounterBytes + (size_t)(n_units * parts) * unit_part_bytes;
            return finish(sp);
        }
    }
    if (!a.causal || n_units > kCUs)
        return finish(sp);
    int64_t total = 0;
    for (int q = 0; q < g.n_qblk; ++q)
        total += tiles(q);
    const int64_t cap = (total + g.n_qblk - 1) / g.n_qblk + kSplitBias;
    int q_split = g.n_qblk;
    while (q_split > 0 && tiles(q_split - 1) > cap)              // tiles grow with the block
        --q_split;
    q_split = std::max(q_split, (g.n_qblk + 1) / 2);             // every split unit's mirror is light
    const int64_t n_split = (int64_t)(g.n_qblk - q_split) * per;
    if (n_split == 0 || n_split * sizeof(uint32_t) > kSplitCounterBytes || cap < 1)
        return finish(sp);
    sp.q_split = q_split;
    sp.cap = (int)cap;
    sp.n_main = (int64_t)g.n_qblk * per;
    sp.n_tail = n_split;
    sp.workspace_bytes = kSplitCounterBytes + (size_t)n_split * 2 * unit_part_bytes;
    return finish(sp);
}

PrefillGrid prefill16_grid(const AttnArgs &a)
{
    PrefillGrid g;
    g.waves = kNW;
    g.hpw = a.G < kNW ? a.G : kNW;
    g.qsub = kNW / g.hpw;
    g.n_qblk = (a.Sq + kQW * g.qsub - 1) / (kQW * g.qsub);
    g.n_hchunk = (a.G + g.hpw - 1) / g.hpw;
    g.n_wg = (int64_t)g.n_qblk * g.n_hchunk * a.Hkv * a.B;
    return g;
}

// every cache type takes this kernel (q4_0: raw LDS-DMA, dequantized into its f16 rings)
PrefillGrid prefill_grid(const AttnArgs &a) { return prefill16_grid(a); }

hipError_t launch_prefill(const AttnArgs &a, hipStream_t stream, const PagedKV *paged,
                          const int32_t *q_lens, int32_t *stats)
{
    const PrefillGrid g = prefill16_grid(a);
    return g.n_wg == 0 ? hipSuccess : launch_prefill16(a, g, stream, paged, q_lens, stats);
}

hipError_t launch_prefill_split(const AttnArgs &a0, const PrefillSplit &sp, void *workspace,
                                hipStream_t stream)
{
    const PrefillGrid g = prefill16_grid(a0);
    if (g.n_wg == 0)
        return hipSuccess;
    AttnArgs a = a0;
    if (sp.deq) {
        // widen the q4_0 tensors into the workspace, then run the 16-bit kernel on the copies
        uint8_t *copy = (uint8_t *)workspace + sp.deq_off;
        const int64_t n_blocks = (int64_t)a0.B * a0.Sk * a0.Hkv * (a0.D / 32);
        if (sp.deq & 1) {
            const hipError_t e = launch_dequant_q4_0(a0.k, n_blocks, nullptr, copy, stream);
            if (e != hipSuccess)
                return e;
            a.k = copy;
            copy += sp.deq_bytes;
        }
        if (sp.deq & 2) {
            const hipError_t e = launch_dequant_q4_0(a0.v, n_blocks, nullptr, copy, stream);
            if (e != hipSuccess)
                return e;
            a.v = copy;
        }
        a.kv = KV_F16;
    }
    if (sp.n_tail == 0)
        return launch_prefill16(a, g, stream);
    Prefill16Params p{a, g.hpw, g.qsub, g.n_qblk, g.n_hchunk, nullptr, nullptr, nullptr, 0, 0};
    p.q_split = sp.q_split;
    p.cap = sp.cap;
    p.n_main = (int)sp.n_main;
    p.n_tail = (int)sp.n_tail;
    p.parts = sp.parts;
    p.cnt = (uint32_t *)workspace;
    p.part = (float *)((uint8_t *)workspace + kSplitCounterBytes);
    return a.D == 128 ? launch16_kv<128>(p, g.n_wg, stream) : launch16_kv<64>(p, g.n_wg, stream);
}

hipError_t launch_prefill16(const AttnArgs &a, const PrefillGrid &g, hipStream_t stream,
                            const PagedKV *paged, const int32_t *q_lens, int32_t *stats)
{
    Prefill16Params p{a, g.hpw, g.qsub, g.n_qblk, g.n_hchunk, nullptr, nullptr, nullptr, 0, 0};
    p.stats = stats;
    if (paged) {
        if (paged->max_pages > kPrefillMaxPages || !paged->block_table || !paged->seq_lens)
            return hipErrorInvalidValue;
        p.block_table = paged->block_table;
        p.seq_lens = paged->seq_lens;
        p.q_lens = q_lens;
        p.max_pages = paged->max_pages;
        p.n_pages = paged->n_pages;
    }
    return a.D == 128 ? launch16_kv<128>(p, g.n_wg, stream) : launch16_kv<64>(p, g.n_wg, stream);
}

#undef INL

}  // namespace fa
