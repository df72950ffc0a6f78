// Device building blocks shared by the prefill, decode and dequant kernels (gfx950 only).
//
// Element values travel as raw 16-bit patterns (uint32 pairs, 16-byte quads) and are
// reinterpreted as f16 or bf16 vectors only at the MFMA and conversion instructions, so one
// code path serves both 16-bit types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// cache types; the last two are mixed (K type, V type): f16 K with q4_0 V and the reverse
enum { KV_F16 = 0, KV_BF16 = 1, KV_Q4_0 = 2, KV_F16_Q4_0 = 3, KV_Q4_0_F16 = 4 };
// K's and V's own types (KV_F16, KV_BF16 or KV_Q4_0)
__host__ __device__ constexpr int kv_k(int kv)
{
    return kv == KV_F16_Q4_0 ? KV_F16 : kv == KV_Q4_0_F16 ? KV_Q4_0 : kv;
}
__host__ __device__ constexpr int kv_v(int kv)
{
    return kv == KV_F16_Q4_0 ? KV_Q4_0 : kv == KV_Q4_0_F16 ? KV_F16 : kv;
}
// bytes of one key row of one head: D 16-bit values, or D/32 q4_0 blocks of 18 bytes
__host__ __device__ constexpr int kv_row_bytes(int t, int D)
{
    return t == KV_Q4_0 ? D / 32 * 18 : 2 * D;
}

// Softmax works in base 2: scores are multiplied by scale*log2(e) and exponentiated with
// v_exp_f32. The rescale margin of 10 natural-log units becomes 10*log2(e).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleMargin = 10.0f;
constexpr float kRescaleMarginLog2 = kRescaleMargin * kLog2e;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------
// MFMA: D = A * B + C with 8 16-bit elements of A and of B per lane.
//   32x32x16: lane l holds A[m = l%32][k = 8*(l/32) .. +7], B[k = 8*(l/32) .. +7][n = l%32];
//             C reg i holds C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32].
//   16x16x32: lane l holds A[m = l%16][k = 8*(l/16) .. +7], B[k = 8*(l/16) .. +7][n = l%16];
//             C reg i holds C[m = 4*(l/16) + i][n = l%16].
// Only the C layout matters for correctness here: the k order inside A and B is the same
// function of (lane, slot) for both operands, so any k permutation cancels in the sum.
// ---------------------------------------------------------------------------------------
template <bool BF>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 16x16x16 with 4 elements per lane: A[m = l%16][k = 4*(l/16) .. +3], B likewise.
template <bool BF>
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a) ,
                                                        __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Two f32 -> packed 16-bit pair, round to nearest even.
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (BF) {
        bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2 v = __builtin_convertvector((f32x2){lo, hi}, f16x2);
        return __builtin_bit_cast(uint32_t, v);
    }
}

// Packed 16-bit pair -> two f32 (exact).
template <bool BF>
__device__ __forceinline__ f32x2 unpack2(uint32_t pair)
{
    if constexpr (BF)
        return __builtin_convertvector(__builtin_bit_cast(bf16x2, pair), f32x2);
    else
        return __builtin_convertvector(__builtin_bit_cast(f16x2, pair), f32x2);
}

// Sum of a packed 16-bit pair, accumulated in f32 (v_dot2 with ones).
template <bool BF>
__device__ __forceinline__ float sum2(uint32_t pair, float acc)
{
    if constexpr (BF) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
    } else {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
    }
}

// Make the compiler treat `x` as read here, so that the wait for its global load is placed
// here and not inside a later loop (where an in-order wait on it would also wait for every
// load issued after it, e.g. the next tile's).
__device__ __forceinline__ void settle(const u32x4 &x) { asm volatile("" ::"v"(x)); }

// max / sum of x over the lane pair {l, l ^ 32}. v_permlane32_swap on two copies of x leaves,
// in every lane, the value of lane l % 32 in one and of lane l % 32 + 32 in the other — a VALU
// exchange, no LDS trip. It is issued from asm: given one value for both operands, the
// compiler's builtin treats its two results as equal and drops one of them. The s_nop covers
// the two wait states the swap needs after a VALU write of its operands.
__device__ __forceinline__ void lane_halves(float x, float &lo, float &hi)
{
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    lo = a;
    hi = b;
}
// f32 maxima as single instructions (v_maximum3_f32). The compiler's fmaxf first quiets every
// operand it cannot prove canonical (MFMA results issued from asm, DPP results: one extra
// v_max_f32 each); the IEEE maximum needs no quieting. The values maximised here are scores and
// their maxima, never NaN (masked keys are -inf), where the two agree.
__device__ __forceinline__ float vmax(float a, float b)
{
    return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ __forceinline__ float pair_max(float x)
{
    float lo, hi;
    lane_halves(x, lo, hi);
    return vmax(lo, hi);
}
__device__ __forceinline__ float pair_sum(float x)
{
    float lo, hi;
    lane_halves(x, lo, hi);
    return lo + hi;
}

// Byte permute: result byte i = byte sel_i of {hi:lo} (0..3 lo, 4..7 hi, 0x0C -> 0).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---------------------------------------------------------------------------------------
// q4_0 unpacking. A code byte holds element t (low nibble) and element t+16 (high nibble)
// of its 32-element block; value (c - 8) * d with the block's f16 scale d.
//
// A nibble c placed in the low mantissa bits of the f16 pattern 0x6400 (= 1024) gives the
// f16 value 1024 + c; subtracting 1032 is exact and leaves c - 8; one f16 multiply by d
// then rounds the exact product (c - 8) * d to nearest even — the same value as the
// correctly rounded f16 of the exact product.
// ---------------------------------------------------------------------------------------
// Two nibbles at bits 0..3 and 16..19 of `nib` -> packed f16 pair (c0 - 8) * d0, (c1 - 8) * d1.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits)
{
    // (x & mask) | bits in one instruction (the compiler otherwise emits an AND and an OR);
    // one scalar operand at most, so `bits` sits in a VGPR
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bits));
    return r;
}

__device__ __forceinline__ uint32_t q4_pair(uint32_t nib, uint32_t d2)
{
    const f16x2 x = __builtin_bit_cast(f16x2, and_or(nib, 0x000F000Fu, 0x64006400u));
    const f16x2 c = x - (f16x2){(_Float16)1032.0f, (_Float16)1032.0f};
    return __builtin_bit_cast(uint32_t, c * __builtin_bit_cast(f16x2, d2));
}

// Four code bytes of one block (bytes 4g .. 4g+3) -> natural-order element pairs:
//   lo[0] = (e[4g], e[4g+1]), lo[1] = (e[4g+2], e[4g+3]),
//   hi[0] = (e[16+4g], e[16+4g+1]), hi[1] = (e[16+4g+2], e[16+4g+3]).
// d2 = the block scale in both halves.
__device__ __forceinline__ void q4_unpack_row(uint32_t codes, uint32_t d2, uint32_t lo[2],
                                              uint32_t hi[2])
{
    const uint32_t u0 = perm(0u, codes, 0x0C010C00u);   // [B0, 0, B1, 0]
    const uint32_t u1 = perm(0u, codes, 0x0C030C02u);   // [B2, 0, B3, 0]
    lo[0] = q4_pair(u0, d2);
    hi[0] = q4_pair(u0 >> 4, d2);
    lo[1] = q4_pair(u1, d2);
    hi[1] = q4_pair(u1 >> 4, d2);
}

// Code byte j of two keys' blocks (c0 for key 0, c1 for key 1) -> key-pairs of one element:
//   lo = (x0[t], x1[t]) and hi = (x0[t+16], x1[t+16]) with t = 4g + j;
// d2 = (d of key 0, d of key 1).
template <int J>
__device__ __forceinline__ void q4_unpack_cols(uint32_t c0, uint32_t c1, uint32_t d2,
                                               uint32_t &lo, uint32_t &hi)
{
    constexpr uint32_t sel = 0x0C000C00u | ((4u + J) << 16) | (uint32_t)J;
    const uint32_t u = perm(c1, c0, sel);                 // [c0.Bj, 0, c1.Bj, 0]
    lo = q4_pair(u, d2);
    hi = q4_pair(u >> 4, d2);
}

// Read the 18-byte block starting `misalign` (0 or 2) bytes into five aligned dwords w[0..4]:
// returns its scale (f16 bits in the low half) and its 16 code bytes as 4 dwords.
__device__ __forceinline__ void q4_split_block(const uint32_t w[5], uint32_t misalign,
                                               uint32_t &d_bits, uint32_t codes[4])
{
    // misalign == 0: scale = w0[15:0], codes start at byte 2 (straddling dwords);
    // misalign == 2: scale = w0[31:16], codes are w1..w4.
    const uint32_t sh = misalign ? 0u : 16u;
    d_bits = (misalign ? (w[0] >> 16) : w[0]) & 0xFFFFu;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t lo = misalign ? w[g + 1] : w[g];
        codes[g] = __builtin_amdgcn_alignbit(w[g + 1], lo, sh);
    }
}

// Data that another workgroup reads in the same launch moves by device-scope (sc1) accesses,
// which bypass the non-coherent per-CU and per-XCD caches: a store is complete once it has
// reached the device's coherence point, and a load reads from there. A workgroup then only
// has to wait for its stores to complete before it counts itself in (arrive_last); no
// whole-L2 write-back or invalidate is needed. Pairs of floats (8-byte aligned) move as one
// 8-byte access.
__device__ __forceinline__ void store_through2(float *p, float x, float y)
{
    const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, x) |
                       ((uint64_t)__builtin_bit_cast(uint32_t, y) << 32);
    __hip_atomic_store((uint64_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_through2(const float *p)
{
    const uint64_t v =
        __hip_atomic_load((const uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__builtin_bit_cast(float, (uint32_t)v),
                 __builtin_bit_cast(float, (uint32_t)(v >> 32))};
}

// Called by every thread of the workgroup after its store_through2 writes; true, in all of
// them, for the workgroup that is the n-th to arrive at counter c, which also returns the
// counter to zero. No workgroup waits for another.
__device__ __forceinline__ bool arrive_last(uint32_t *c, uint32_t n, uint32_t *flag)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t last = old + 1 == n ? 1u : 0u;
        if (last)
            __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    const bool last = *flag != 0;
    asm volatile("" ::: "memory");
    return last;
}

// Grid remap so that consecutive logical workgroups run on the same XCD: the hardware deals
// workgroup ids round-robin over the 8 XCDs, so id -> (id % 8) * (n / 8) + id / 8 hands each
// XCD one contiguous slice of the logical order (and so of K/V heads, which share its L2).
__device__ __forceinline__ int xcd_remap(int id, int n)
{
    if (n % 8)
        return id;
    return (id % 8) * (n / 8) + id / 8;
}

}  // namespace fa
