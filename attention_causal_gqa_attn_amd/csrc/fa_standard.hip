// Standard (non-flash) attention: the comparison arm of mi210-llm-stack, "FlashAttention on
// gfx90a", "Three Patching Approaches" (Approach C) and "The V Dequantization Gap". That page
// names the non-FA path of its stack as the fast one on its GPU and the fix as dequantizing V in
// that path the way K already is. Here the path is, per (b, KV head) unit:
//
//   1. a q4_0 K or V cache is dequantized to f16 (the same routine fa_dequant_q4_0 runs);
//   2. S = scale * Q K^T, materialised in f32 for every (query row, key) tile that holds a
//      visible pair (MFMA, 128 x 128 tiles);
//   3. a row softmax over the visible keys writes P = exp(S - max) / sum in the Q type, zero
//      past the row's last visible key;
//   4. O = P V (MFMA, 128-row tiles, 64-key steps; split over the keys into f32 partials and
//      summed by a last kernel when the rows alone give too few workgroups, as in decode).
//
// Rows of a unit are the G query heads of each query, r = i * G + hh. Every step reads and
// writes HBM in full, which is what the flash kernels avoid; this path exists to be timed
// beside them, not to be fast.
#include "fa_kernels.h"
#include "fa_device.h"

namespace fa {

namespace {

constexpr int kSB = 128;   // rows and keys of a score tile; rows of an output tile
constexpr int kPK = 64;    // keys per P.V step
constexpr int kTh = 256;   // threads per workgroup (4 waves)
constexpr int kPvTarget = 512;   // P.V workgroups wanted (two per CU)

struct StdParams {
    AttnArgs a;
    float scale;
    const uint16_t *k16, *v16;   // 16-bit K and V ([B, Sk, Hkv, D]; dequantized copies for q4_0)
    float *S;                    // [unit of the pass][rows_g][Skp] f32
    uint16_t *P;                 // [unit of the pass][rows_g][Skp], the Q type
    float *Opart;                // [split][unit of the pass][rows_g][D] f32 (nks > 1)
    int64_t Skp;                 // padded row length, a multiple of kSB
    int rows_g;                  // Sq * G rows per unit
    int unit0, n_units;          // this pass: units [unit0, unit0 + n_units) of B * Hkv
    int n_rtile, n_ktile;        // row tiles per unit, key tiles per row
    int nks, ks_len;             // P.V key splits, keys per split (a multiple of kPK)
};

// keys row query i can see: [0, nvis)
__device__ __forceinline__ int64_t nvis(const AttnArgs &a, int i)
{
    if (!a.causal)
        return a.Sk;
    const int64_t e = (int64_t)i + a.offset + 1;
    return e < 0 ? 0 : (e > a.Sk ? (int64_t)a.Sk : e);
}

// Q (or O) row r of unit (b, kvh): query i = r / G of head kvh * G + r % G
__device__ __forceinline__ int64_t row_elem(const AttnArgs &a, int b, int kvh, int r)
{
    const int i = r / a.G, hh = r % a.G;
    return (((int64_t)b * a.Sq + i) * a.Hq + kvh * a.G + hh) * a.D;
}

// 16-byte chunk c of row x of an LDS tile with W-byte rows, swizzled so that 32 lanes reading
// one chunk column of consecutive rows spread over the banks
template <int W>
__device__ __forceinline__ int swz(int x, int c)
{
    constexpr int C = W / 16;
    return x * W + 16 * (c ^ (x & (C - 1)));
}

// ---- 2. scores ----------------------------------------------------------------------------------
template <int D, bool BF>
__global__ __launch_bounds__(kTh, 2) void std_qk_kernel(StdParams p)
{
    constexpr int CPR = D / 8, ROWB = 2 * D;
    __shared__ __attribute__((aligned(16))) uint8_t lq[kSB * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t lk[kSB * ROWB];
    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int rest = blockIdx.x;
    const int kt = rest % p.n_ktile;
    rest /= p.n_ktile;
    const int rt = rest % p.n_rtile;
    const int ul = rest / p.n_rtile;                 // unit within the pass
    const int u = p.unit0 + ul, b = u / a.Hkv, kvh = u % a.Hkv;
    const int r0 = rt * kSB, j0 = kt * kSB;
    const int rlast = min(r0 + kSB, p.rows_g) - 1;
    if ((int64_t)j0 >= nvis(a, rlast / a.G))
        return;                                      // no row of the tile sees these keys

    for (int e = t; e < kSB * CPR; e += kTh) {
        const int x = e / CPR, c = e % CPR;
        const uint16_t *qp = (const uint16_t *)a.q + row_elem(a, b, kvh, min(r0 + x, p.rows_g - 1));
        const int j = min(j0 + x, a.Sk - 1);
        const uint16_t *kp = p.k16 + (((int64_t)b * a.Sk + j) * a.Hkv + kvh) * D;
        *(u32x4 *)(lq + swz<ROWB>(x, c)) = *(const u32x4 *)(qp + 8 * c);
        *(u32x4 *)(lk + swz<ROWB>(x, c)) = *(const u32x4 *)(kp + 8 * c);
    }
    __syncthreads();

    // wave tile: rows 64 (wave / 2) .. +63, keys 64 (wave % 2) .. +63, as 2 x 2 MFMA tiles
    const int wr = 64 * (wave >> 1), wc = 64 * (wave & 1), m = lane & 31, kh = lane >> 5;
    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
            acc[x][y] = (f32x16){};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const int c = 2 * s + kh;
        u32x4 af[2], bf[2];
#pragma unroll
        for (int x = 0; x < 2; ++x)
            af[x] = *(const u32x4 *)(lq + swz<ROWB>(wr + 32 * x + m, c));
#pragma unroll
        for (int y = 0; y < 2; ++y)
            bf[y] = *(const u32x4 *)(lk + swz<ROWB>(wc + 32 * y + m, c));
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
                acc[x][y] = mfma32<BF>(af[x], bf[y], acc[x][y]);
    }

    // C register i: row 8 (i / 4) + 4 kh + i % 4 of the 32-row tile, key m
    float *Sb = p.S + (int64_t)ul * p.rows_g * p.Skp;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = r0 + wr + 32 * x + 8 * (i / 4) + 4 * kh + (i % 4);
            if (r < p.rows_g) {
#pragma unroll
                for (int y = 0; y < 2; ++y)
                    Sb[(int64_t)r * p.Skp + j0 + wc + 32 * y + m] = acc[x][y][i] * p.scale;
            }
        }
}

// ---- 3. row softmax -----------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float x, bool is_max, float *red)
{
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) {
        const float y = __shfl_xor(x, sh, 64);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int t = threadIdx.x;
    __syncthreads();
    if ((t & 63) == 0)
        red[t >> 6] = x;
    __syncthreads();
    x = red[0];
#pragma unroll
    for (int w = 1; w < kTh / 64; ++w)
        x = is_max ? fmaxf(x, red[w]) : x + red[w];
    return x;
}

template <bool BF>
__global__ __launch_bounds__(kTh) void std_softmax_kernel(StdParams p)
{
    __shared__ float red[kTh / 64];
    const AttnArgs &a = p.a;
    const int64_t row = blockIdx.x;                  // (unit of the pass) * rows_g + r
    const int r = (int)(row % p.rows_g);
    const int64_t n = nvis(a, r / a.G);
    const float *s = p.S + row * p.Skp;
    uint16_t *P = p.P + row * p.Skp;
    const int t = threadIdx.x;

    float mx = -INFINITY;
    for (int64_t j = 4 * t; j < n; j += 4 * kTh) {
        const f32x4 x = *(const f32x4 *)(s + j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e < n)
                mx = fmaxf(mx, x[e]);
    }
    mx = block_reduce(mx, true, red);
    float l = 0.0f;
    for (int64_t j = 4 * t; j < n; j += 4 * kTh) {
        const f32x4 x = *(const f32x4 *)(s + j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e < n)
                l += expf(x[e] - mx);
    }
    l = block_reduce(l, false, red);
    for (int64_t j = 4 * t; j < p.Skp; j += 4 * kTh) {
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (j < n) {
            const f32x4 x = *(const f32x4 *)(s + j);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < n)
                    v[e] = expf(x[e] - mx) / l;
        }
        *(u32x2 *)(P + j) = (u32x2){pack2<BF>(v[0], v[1]), pack2<BF>(v[2], v[3])};
    }
}

// ---- 4. O = P V ---------------------------------------------------------------------------------
template <int D, bool BF>
__global__ __launch_bounds__(kTh, 2) void std_pv_kernel(StdParams p)
{
    constexpr int WR = D == 128 ? 2 : 4;             // waves along rows
    constexpr int WC = 4 / WR;                       // waves along d
    constexpr int TR = kSB / WR / 32;                // 32-row MFMA tiles per wave
    constexpr int TC = D / WC / 32;                  // 32-column MFMA tiles per wave
    constexpr int PW = 2 * kPK;                      // bytes of a P tile row and a V^T row
    __shared__ __attribute__((aligned(16))) uint8_t lp[kSB * PW];   // P [row][key]
    __shared__ __attribute__((aligned(16))) uint8_t lv[D * PW];     // V^T [d][key]
    const AttnArgs &a = p.a;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int rest = blockIdx.x;
    const int ks = rest % p.nks;
    rest /= p.nks;
    const int rt = rest % p.n_rtile;
    const int ul = rest / p.n_rtile;
    const int u = p.unit0 + ul, b = u / a.Hkv, kvh = u % a.Hkv;
    const int r0 = rt * kSB;
    const int rlast = min(r0 + kSB, p.rows_g) - 1;
    const int64_t kend = nvis(a, rlast / a.G);
    const int64_t kbeg = (int64_t)ks * p.ks_len;
    const int64_t kstop = min(kend, kbeg + p.ks_len);
    const uint16_t *Pb = p.P + (int64_t)ul * p.rows_g * p.Skp;

    const int wr = (kSB / WR) * (wave / WC), wc = (D / WC) * (wave % WC);
    const int m = lane & 31, kh = lane >> 5;
    f32x16 acc[TR][TC];
#pragma unroll
    for (int x = 0; x < TR; ++x)
#pragma unroll
        for (int y = 0; y < TC; ++y)
            acc[x][y] = (f32x16){};

    for (int64_t k0 = kbeg; k0 < kstop; k0 += kPK) {
        __syncthreads();                             // every wave is done with the last step
        // P tile: 128 rows x 8 chunks (keys k0 .. k0 + 63 < Skp: P is zero past a row's keys)
        for (int e = t; e < kSB * (kPK / 8); e += kTh) {
            const int x = e / (kPK / 8), c = e % (kPK / 8);
            const int64_t rr = min(r0 + x, p.rows_g - 1);
            *(u32x4 *)(lp + swz<PW>(x, c)) = *(const u32x4 *)(Pb + rr * p.Skp + k0 + 8 * c);
        }
        // V^T tile: 8 x 8 blocks (8 keys x 8 d) transposed through registers
        for (int blk = t; blk < (kPK / 8) * (D / 8); blk += kTh) {
            const int kb = blk / (D / 8), dc = blk % (D / 8);
            u32x4 in[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t j = min(k0 + 8 * kb + e, (int64_t)a.Sk - 1);
                in[e] = *(const u32x4 *)(p.v16 + ((b * (int64_t)a.Sk + j) * a.Hkv + kvh) * D + 8 * dc);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = perm(in[2 * q + 1][c >> 1], in[2 * q][c >> 1], sel);
                *(u32x4 *)(lv + swz<PW>(8 * dc + c, kb)) = o;
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kPK / 16; ++s) {
            const int c = 2 * s + kh;
            u32x4 af[TR], bf[TC];
#pragma unroll
            for (int x = 0; x < TR; ++x)
                af[x] = *(const u32x4 *)(lp + swz<PW>(wr + 32 * x + m, c));
#pragma unroll
            for (int y = 0; y < TC; ++y)
                bf[y] = *(const u32x4 *)(lv + swz<PW>(wc + 32 * y + m, c));
#pragma unroll
            for (int x = 0; x < TR; ++x)
#pragma unroll
                for (int y = 0; y < TC; ++y)
                    acc[x][y] = mfma32<BF>(af[x], bf[y], acc[x][y]);
        }
    }

    // C register i: row 8 (i / 4) + 4 kh + i % 4, column (d) m
#pragma unroll
    for (int x = 0; x < TR; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = r0 + wr + 32 * x + 8 * (i / 4) + 4 * kh + (i % 4);
            if (r >= p.rows_g)
                continue;
#pragma unroll
            for (int y = 0; y < TC; ++y) {
                const int d = wc + 32 * y + m;
                if (p.nks == 1) {
                    uint16_t *op = (uint16_t *)a.o + row_elem(a, b, kvh, r);
                    op[d] = (uint16_t)(pack2<BF>(acc[x][y][i], 0.0f) & 0xFFFFu);
                } else {
                    p.Opart[(((int64_t)ks * p.n_units + ul) * p.rows_g + r) * D + d] =
                        acc[x][y][i];
                }
            }
        }
}

// Sum of the P.V key splits of each output element.
template <int D, bool BF>
__global__ __launch_bounds__(kTh) void std_pv_sum_kernel(StdParams p)
{
    const AttnArgs &a = p.a;
    const int64_t e = (int64_t)blockIdx.x * kTh + threadIdx.x;   // (unit, r, d)
    const int64_t per_split = (int64_t)p.n_units * p.rows_g * D;
    if (e >= per_split)
        return;
    float sum = 0.0f;
    for (int ks = 0; ks < p.nks; ++ks)
        sum += p.Opart[(int64_t)ks * per_split + e];
    const int d = (int)(e % D);
    const int64_t ur = e / D;
    const int r = (int)(ur % p.rows_g), ul = (int)(ur / p.rows_g);
    const int u = p.unit0 + ul;
    uint16_t *op = (uint16_t *)a.o + row_elem(a, u / a.Hkv, u % a.Hkv, r);
    op[d] = (uint16_t)(pack2<BF>(sum, 0.0f) & 0xFFFFu);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct StdPlan {
    int64_t Skp;
    int rows_g, n_rtile, n_ktile, units, upp, nks, ks_len;
    size_t kcopy, vcopy, s_bytes, p_bytes, opart_bytes, total;
};

// Layout of the workspace for upp units per pass.
StdPlan std_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv, int upp)
{
    StdPlan pl{};
    pl.Skp = ((int64_t)(Sk > 0 ? Sk : 1) + kSB - 1) / kSB * kSB;
    pl.rows_g = Sq * (Hq / Hkv);
    pl.n_rtile = (pl.rows_g + kSB - 1) / kSB;
    pl.n_ktile = (int)(pl.Skp / kSB);
    pl.units = B * Hkv;
    pl.upp = upp <= 0 || upp > pl.units ? pl.units : upp;
    const int64_t groups = (int64_t)pl.upp * pl.n_rtile;
    const int64_t steps = (Sk + kPK - 1) / kPK;
    int64_t nks = groups >= kPvTarget ? 1 : (kPvTarget + groups - 1) / groups;
    nks = nks > steps ? (steps > 0 ? steps : 1) : nks;
    const int64_t per = (steps + nks - 1) / nks;
    pl.ks_len = (int)((per > 0 ? per : 1) * kPK);
    pl.nks = (int)(steps > 0 ? (steps + per - 1) / per : 1);
    const size_t kvelems = (size_t)B * Sk * Hkv * D;
    pl.kcopy = kv_k(kv) == KV_Q4_0 ? align256(kvelems * 2) : 0;
    pl.vcopy = kv_v(kv) == KV_Q4_0 ? align256(kvelems * 2) : 0;
    const size_t rows = (size_t)pl.upp * pl.rows_g;
    pl.s_bytes = align256(rows * pl.Skp * 4);
    pl.p_bytes = align256(rows * pl.Skp * 2);
    pl.opart_bytes = pl.nks > 1 ? align256((size_t)pl.nks * rows * D * 4) : 0;
    pl.total = pl.kcopy + pl.vcopy + pl.s_bytes + pl.p_bytes + pl.opart_bytes;
    return pl;
}

template <int D, bool BF>
hipError_t std_pass(const StdParams &p, hipStream_t stream)
{
    const int64_t nqk = (int64_t)p.n_units * p.n_rtile * p.n_ktile;
    hipLaunchKernelGGL((std_qk_kernel<D, BF>), dim3((unsigned)nqk), dim3(kTh), 0, stream, p);
    hipLaunchKernelGGL((std_softmax_kernel<BF>), dim3((unsigned)((int64_t)p.n_units * p.rows_g)),
                       dim3(kTh), 0, stream, p);
    const int64_t npv = (int64_t)p.n_units * p.n_rtile * p.nks;
    hipLaunchKernelGGL((std_pv_kernel<D, BF>), dim3((unsigned)npv), dim3(kTh), 0, stream, p);
    if (p.nks > 1) {
        const int64_t n = (int64_t)p.n_units * p.rows_g * D;
        hipLaunchKernelGGL((std_pv_sum_kernel<D, BF>), dim3((unsigned)((n + kTh - 1) / kTh)),
                           dim3(kTh), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

size_t standard_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv,
                                int units_per_pass)
{
    return std_plan(B, Hq, Hkv, Sq, Sk, D, kv, units_per_pass).total;
}

int64_t standard_max_workgroups(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv)
{
    const StdPlan pl = std_plan(B, Hq, Hkv, Sq, Sk, D, kv, 0);
    const int64_t qk = (int64_t)pl.units * pl.n_rtile * pl.n_ktile;
    const int64_t sm = (int64_t)pl.units * pl.rows_g;
    return qk > sm ? qk : sm;
}

hipError_t launch_standard(const AttnArgs &a, float scale, void *workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    // all units in one pass if the workspace holds them, else halve until it does (the caller
    // checked that one unit per pass fits)
    int upp = a.B * a.Hkv;
    StdPlan pl = std_plan(a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.D, a.kv, upp);
    while (pl.total > workspace_bytes && upp > 1) {
        upp = upp / 2 > 1 ? upp / 2 : 1;
        pl = std_plan(a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.D, a.kv, upp);
    }
    if (pl.total > workspace_bytes)
        return hipErrorInvalidValue;
    uint8_t *ws = (uint8_t *)workspace;
    StdParams p{};
    p.a = a;
    p.scale = scale;
    p.k16 = (const uint16_t *)a.k;
    p.v16 = (const uint16_t *)a.v;
    const int64_t nblk = (int64_t)a.B * a.Sk * a.Hkv * (a.D / 32);
    if (pl.kcopy) {
        p.k16 = (const uint16_t *)ws;
        const hipError_t e = launch_dequant_q4_0(a.k, nblk, nullptr, ws, stream);
        if (e != hipSuccess)
            return e;
    }
    if (pl.vcopy) {
        p.v16 = (const uint16_t *)(ws + pl.kcopy);
        const hipError_t e = launch_dequant_q4_0(a.v, nblk, nullptr, ws + pl.kcopy, stream);
        if (e != hipSuccess)
            return e;
    }
    p.S = (float *)(ws + pl.kcopy + pl.vcopy);
    p.P = (uint16_t *)(ws + pl.kcopy + pl.vcopy + pl.s_bytes);
    p.Opart = (float *)(ws + pl.kcopy + pl.vcopy + pl.s_bytes + pl.p_bytes);
    p.Skp = pl.Skp;
    p.rows_g = pl.rows_g;
    p.n_rtile = pl.n_rtile;
    p.n_ktile = pl.n_ktile;
    p.nks = pl.nks;
    p.ks_len = pl.ks_len;
    const bool bf = a.kv == KV_BF16;
    for (int u0 = 0; u0 < pl.units; u0 += pl.upp) {
        p.unit0 = u0;
        p.n_units = pl.units - u0 < pl.upp ? pl.units - u0 : pl.upp;
        hipError_t e;
        if (a.D == 128)
            e = bf ? std_pass<128, true>(p, stream) : std_pass<128, false>(p, stream);
        else
            e = bf ? std_pass<64, true>(p, stream) : std_pass<64, false>(p, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace fa
