// K/V tile staging for the decode kernels that keep f16 tiles in LDS (the 16-bit caches, and
// q4_0 with more than 4 query rows per KV head): global memory or a raw LDS stage -> registers
// -> LDS. A tile is kBN = 64 consecutive keys of one KV head:
//   K tile  [64 keys][D]      row stride D + 8 elements (16 B pad: conflict-free row reads)
//   V^T tile [D][64 keys]     row stride 64 + 8 elements (transposed at store time, so the
//                             P.V MFMA reads 8 consecutive keys of one d as one 16-byte load)
// Both hold f16 or bf16 values; a q4_0 cache is dequantized on the way into LDS, so the
// MFMA loop is the same for every cache type.
//
// Work split over the 256 threads of a workgroup:
//   16-bit K: 16-byte chunks, id = pass * 256 + t -> key id / (D/8), chunk id % (D/8).
//   16-bit V: KPT = D/32 consecutive keys x one 16-byte chunk per thread; the KPT rows are
//             transposed in registers with byte permutes and written as KPT-key runs.
//   q4_0:     one item = 2 consecutive keys x 1 block; threads [0, D) take K, [D, 2D) take V.
//   mixed (one f16 and one q4_0 cache): the f16 loader's half for the f16 tensor, the q4_0
//             loader's threads for the other.
// Key indices past the end of the sequence are clamped to the last key: those slots are
// masked out of the softmax, and clamping keeps every load in bounds and every value finite.
#pragma once

#include "fa_device.h"

namespace fa {

constexpr int kBN = 64;          // keys per tile
constexpr int kThreads = 256;    // threads per workgroup

template <int D>
struct TileGeom {
    static constexpr int kStride = D + 8;
    static constexpr int vStride = kBN + 8;
    static constexpr int kElems = kBN * kStride;
    static constexpr int vElems = D * vStride;
    static constexpr int stage = kElems + vElems;     // 16-bit elements per K+V buffer
};

// NT: threads of the workgroup that stages the tiles (256 or 512).
template <int D, int KV, int NT = kThreads>
struct TileLoader;

// f16 / bf16 caches ----------------------------------------------------------------------
template <int D, int KV, int NT>
struct TileLoader {
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(NT == 256 || NT == 512, "threads");
    using G = TileGeom<D>;
    static constexpr int KC = kBN * (D / 8) / NT;    // K chunks per thread
    static constexpr int KPT = kBN * (D / 8) / NT;   // V keys per thread
    static constexpr int VCOLS = kBN / KPT;

    const uint8_t *kbase, *vbase;         // first byte of (b, key 0, kvh)
    uint32_t row;                         // bytes between consecutive keys
    int Sk, t;
    uint32_t koff, voff;                  // per-thread byte offsets of the first K chunk / V key
    u32x4 kr[KC], vr[KPT];

    // K chunk p of thread t: key p * kKeysPerPass + t / (D/8), 16-byte chunk t % (D/8)
    static constexpr int kKeysPerPass = NT / (D / 8);
    __device__ __forceinline__ int k_key(int p) const { return p * kKeysPerPass + t / (D / 8); }
    __device__ __forceinline__ int k_dc() const { return t % (D / 8); }
    __device__ __forceinline__ int v_key0() const { return KPT * (t % VCOLS); }
    __device__ __forceinline__ int v_dc() const { return t / VCOLS; }

    // head_off_rows: key-row index of (b, key 0, kvh); row_rows: key rows between keys (Hkv)
    __device__ void init(const void *k, const void *v, int64_t head_off_rows, int64_t row_rows,
                         int Sk_, int t_)
    {
        kbase = (const uint8_t *)k + head_off_rows * D * 2;
        vbase = (const uint8_t *)v + head_off_rows * D * 2;
        row = (uint32_t)(row_rows * D * 2);
        Sk = Sk_;
        t = t_;
        koff = (uint32_t)k_key(0) * row + (uint32_t)k_dc() * 16u;
        voff = (uint32_t)v_key0() * row + (uint32_t)v_dc() * 16u;
    }

    // Global loads of the K (V) tile starting at key k0 (k0 < Sk), whose key-0 row is toff
    // bytes past the head's (k0 rows on in a contiguous cache, its page in a paged one): a
    // uniform tile base plus a 32-bit offset (the per-pass / per-key part of it is uniform, the
    // per-thread part fixed), both branches in 32 bits so the loads keep the scalar-base form
    // after the compiler merges them. In the last, partial tile keys past the end repeat the
    // last key.
    __device__ __forceinline__ void load_k(int k0, int64_t toff)
    {
        const uint8_t *kt = kbase + toff;
        if (k0 + kBN <= Sk) {
#pragma unroll
            for (int p = 0; p < KC; ++p)
                kr[p] = *(const u32x4 *)(kt + ((uint32_t)(p * kKeysPerPass) * row + koff));
        } else {
            const int last = Sk - 1 - k0;
#pragma unroll
            for (int p = 0; p < KC; ++p) {
                const uint32_t off = (uint32_t)min(k_key(p), last) * row + (uint32_t)k_dc() * 16u;
                kr[p] = *(const u32x4 *)(kt + off);
            }
        }
    }

    __device__ __forceinline__ void load_v(int k0, int64_t toff)
    {
        const uint8_t *vt = vbase + toff;
        if (k0 + kBN <= Sk) {
#pragma unroll
            for (int r = 0; r < KPT; ++r)
                vr[r] = *(const u32x4 *)(vt + ((uint32_t)r * row + voff));
        } else {
            const int last = Sk - 1 - k0;
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                const uint32_t off =
                    (uint32_t)min(v_key0() + r, last) * row + (uint32_t)v_dc() * 16u;
                vr[r] = *(const u32x4 *)(vt + off);
            }
        }
    }

    __device__ __forceinline__ void load(int k0, int64_t toff)
    {
        load_k(k0, toff);
        load_v(k0, toff);
    }
    // K and V tile offsets apart (they differ when the two caches have different row sizes)
    __device__ __forceinline__ void load(int k0, int64_t tk, int64_t tv)
    {
        load_k(k0, tk);
        load_v(k0, tv);
    }

    __device__ __forceinline__ void store_k(uint16_t *lk) const
    {
#pragma unroll
        for (int p = 0; p < KC; ++p)
            *(u32x4 *)(lk + k_key(p) * G::kStride + k_dc() * 8) = kr[p];
    }

    __device__ __forceinline__ void store_v(uint16_t *lv) const
    {
        const int key0 = v_key0(), dc = v_dc();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            uint16_t *dst = lv + (dc * 8 + e) * G::vStride + key0;
            if constexpr (KPT == 4) {
                u32x2 w;
                w[0] = perm(vr[1][e / 2], vr[0][e / 2], sel);
                w[1] = perm(vr[3][e / 2], vr[2][e / 2], sel);
                *(u32x2 *)dst = w;
            } else if constexpr (KPT == 2) {
                *(uint32_t *)dst = perm(vr[1][e / 2], vr[0][e / 2], sel);
            } else {
                *dst = (uint16_t)(vr[0][e / 2] >> (16 * (e & 1)));
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t *lk, uint16_t *lv) const
    {
        store_k(lk);
        store_v(lv);
    }
};

// q4_0 cache -----------------------------------------------------------------------------
template <int D, int NT>
struct TileLoader<D, KV_Q4_0, NT> {
    static_assert(D == 64 || D == 128, "head dim");
    using G = TileGeom<D>;
    static constexpr int NB = D / 32;           // blocks per key row
    static constexpr int ROWB = NB * 18;        // bytes per key row

    // threads [0, D) stage K, [D, 2D) stage V, the rest idle (none at D = 128 with 256 threads)
    static constexpr bool kAllBusy = (2 * D == NT);

    const uint8_t *base;                        // K or V, first byte of (b, key 0, kvh)
    uint32_t row;                               // bytes between consecutive keys
    int Sk, tensor, kp, blk, mis;
    bool active;
    uint32_t off[2];                            // byte offsets of this thread's 2 key rows
    uint32_t bo;                                // its block's offset in a row, rounded to 4
    uint32_t w[2][5];

    __device__ __forceinline__ bool busy() const { return active; }

    // only: -1 both tensors, 0 K only, 1 V only (the other tensor's threads stay idle)
    __device__ void init(const void *k, const void *v, int64_t head_off_rows, int64_t row_rows,
                         int Sk_, int t, int only = -1)
    {
        tensor = t / D;                         // 0: K, 1: V, >= 2: idle
        active = only < 0 ? (kAllBusy || tensor < 2) : tensor == only;
        const int u = t % D;
        kp = u % 32;
        if constexpr (D == 128) {
            // a wave takes the even blocks {0, 2} or the odd blocks {1, 3} of its tensor, so
            // the block's alignment (blocks start at byte 0 or 2 of a dword) is wave-uniform
            const int wi = __builtin_amdgcn_readfirstlane(t >> 6) & 1;
            blk = 2 * ((u >> 5) & 1) + wi;
            mis = 2 * wi;
        } else {
            blk = u / 32;
            mis = (18 * blk) & 3;
        }
        const int boff = 18 * blk;
        base = (const uint8_t *)(tensor ? v : k) + head_off_rows * ROWB;
        row = (uint32_t)(row_rows * ROWB);
        Sk = Sk_;
#pragma unroll
        for (int r = 0; r < 2; ++r)
            off[r] = (uint32_t)(2 * kp + r) * row + (uint32_t)(boff & ~3);
        bo = (uint32_t)(boff & ~3);
    }

    // The raw tile is copied into LDS by 12-byte LDS-DMA
    // transfers, each landing in a 16-byte slot. Chunk j (bytes 12j .. 12j+11) of key row
    // 2*kp + rr sits in slot (rr*32 + kp) * RAW_STRIDE + j: even and odd rows in separate
    // halves and an odd slot stride, so the 16-byte reads of consecutive lanes (consecutive kp)
    // hit distinct LDS banks. A block (18 bytes from 18*blk) spans chunks jA = 18*blk / 12 and
    // jA + 1, starting at byte 0 or 6 of chunk jA.
    static constexpr int RAW_CPR = ROWB / 12;
    static constexpr int RAW_STRIDE = RAW_CPR | 1;
    static constexpr int RAW_SLOTS = 64 * RAW_STRIDE;          // slots of one tensor's tile
    static_assert(ROWB % 12 == 0, "key rows split into 12-byte chunks");
    // The same 5-dword windows from global memory: the tile at key k0, whose key-0 row is toff
    // bytes past the head's (4-byte aligned: rows are a multiple of 4 bytes and a window
    // starts at its block's byte offset rounded down to 4; it never passes the row's end)
    __device__ __forceinline__ void load(int k0, int64_t toff)
    {
        if (!busy())
            return;
        const uint8_t *tb = base + toff;
        const int last = Sk - 1 - k0;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const uint32_t o = (uint32_t)min(2 * kp + rr, last) * row + bo;
#pragma unroll
            for (int i = 0; i < 5; ++i)
                w[rr][i] = *(const uint32_t *)(tb + o + 4 * i);
        }
    }

    __device__ __forceinline__ void load_raw(const uint8_t *rk, const uint8_t *rv)
    {
        if (!busy())
            return;
        const uint8_t *r = tensor ? rv : rk;
        const int ja = (18 * blk) / 12;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const uint8_t *sa = r + 16 * ((rr * 32 + kp) * RAW_STRIDE + ja);
            const u32x4 A = *(const u32x4 *)sa, Bq = *(const u32x4 *)(sa + 16);
            // the 5-dword window of load(): starts at byte 0 of chunk jA (mis 0) or 4 (mis 2)
            if (mis == 0) {
                w[rr][0] = A[0]; w[rr][1] = A[1]; w[rr][2] = A[2];
                w[rr][3] = Bq[0]; w[rr][4] = Bq[1];
            } else {
                w[rr][0] = A[1]; w[rr][1] = A[2]; w[rr][2] = Bq[0];
                w[rr][3] = Bq[1]; w[rr][4] = Bq[2];
            }
        }
    }

    __device__ void store(uint16_t *lk, uint16_t *lv) const
    {
        if (!busy())
            return;
        uint32_t dbits[2], codes[2][4];
        q4_split_block(w[0], mis, dbits[0], codes[0]);
        q4_split_block(w[1], mis, dbits[1], codes[1]);
        if (tensor == 0) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const uint32_t d2 = dbits[r] * 0x10001u;
                uint32_t lo[4][2], hi[4][2];
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    q4_unpack_row(codes[r][g], d2, lo[g], hi[g]);
                uint16_t *dst = lk + (2 * kp + r) * G::kStride + 32 * blk;
                *(u32x4 *)(dst + 0) = (u32x4){lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
                *(u32x4 *)(dst + 8) = (u32x4){lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
                *(u32x4 *)(dst + 16) = (u32x4){hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
                *(u32x4 *)(dst + 24) = (u32x4){hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
            }
        } else {
            const uint32_t d2 = dbits[0] | (dbits[1] << 16);
            uint16_t *col = lv + (32 * blk) * G::vStride + 2 * kp;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t lo, hi;
                q4_unpack_cols<0>(codes[0][g], codes[1][g], d2, lo, hi);
                *(uint32_t *)(col + (4 * g + 0) * G::vStride) = lo;
                *(uint32_t *)(col + (4 * g + 16) * G::vStride) = hi;
                q4_unpack_cols<1>(codes[0][g], codes[1][g], d2, lo, hi);
                *(uint32_t *)(col + (4 * g + 1) * G::vStride) = lo;
                *(uint32_t *)(col + (4 * g + 17) * G::vStride) = hi;
                q4_unpack_cols<2>(codes[0][g], codes[1][g], d2, lo, hi);
                *(uint32_t *)(col + (4 * g + 2) * G::vStride) = lo;
                *(uint32_t *)(col + (4 * g + 18) * G::vStride) = hi;
                q4_unpack_cols<3>(codes[0][g], codes[1][g], d2, lo, hi);
                *(uint32_t *)(col + (4 * g + 3) * G::vStride) = lo;
                *(uint32_t *)(col + (4 * g + 19) * G::vStride) = hi;
            }
        }
    }
};

// mixed caches ---------------------------------------------------------------------------
// QK: K is the q4_0 tensor (V f16), else V is (K f16). Both loaders take the same key-row
// index of the head; each scales it by its own row size.
template <int D, bool QK, int NT>
struct MixedLoader {
    TileLoader<D, KV_F16, NT> f;
    TileLoader<D, KV_Q4_0, NT> q;
    __device__ void init(const void *k, const void *v, int64_t head_off_rows, int64_t row_rows,
                         int Sk, int t)
    {
        f.init(k, v, head_off_rows, row_rows, Sk, t);
        q.init(k, v, head_off_rows, row_rows, Sk, t, QK ? 0 : 1);
    }
    __device__ __forceinline__ void load(int k0, int64_t tk, int64_t tv)
    {
        if constexpr (QK) {
            q.load(k0, tk);
            f.load_v(k0, tv);
        } else {
            f.load_k(k0, tk);
            q.load(k0, tv);
        }
    }
    __device__ __forceinline__ void store(uint16_t *lk, uint16_t *lv) const
    {
        if constexpr (QK) {
            q.store(lk, lv);
            f.store_v(lv);
        } else {
            f.store_k(lk);
            q.store(lk, lv);
        }
    }
};
template <int D, int NT>
struct TileLoader<D, KV_F16_Q4_0, NT> : MixedLoader<D, false, NT> {};
template <int D, int NT>
struct TileLoader<D, KV_Q4_0_F16, NT> : MixedLoader<D, true, NT> {};

}  // namespace fa
