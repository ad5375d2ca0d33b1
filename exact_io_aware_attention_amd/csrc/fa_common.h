// Shared device-side definitions of the gfx950 attention kernels.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64),
// measured on gfx950 with an in-bounds probe:
//   A (32 x 16, rows m, depth k): lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   B (16 x 32, depth k, cols n): lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   C (32 x 32):                   lane l, register r holds
//                                  C[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32]
// The contraction index k may be permuted freely as long as A and B use the
// same permutation; the kernels use this to feed an accumulator (C layout)
// straight back in as a B operand: registers 8h..8h+7 of a C tile become the
// 16-deep k-slice h, with slot s of lane half g standing for row
//   16 h + 8 (s / 4) + 4 g + (s % 4)
// of the C tile.
//
// LDS transpose read (ds_read_b64_tr_b16), measured on gfx950: within each
// group of 16 lanes, lane i receives element (i % 4) of the 8-byte rows
// addressed by lanes 4t + i / 4, t = 0..3. Pointing lane 4t + u of a group at
// row key_t, columns c0 + 4u .. c0 + 4u + 3 of a row-major tile gives lane i
// the four values tile[key_t][c0 + i], t = 0..3: a column slice, i.e. the
// transposed operand, without a transposing copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaskBlock = 128;
constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulating MFMA whose accumulator lives in AGPRs (acc += A B). The
// compiler keeps values an MFMA builtin produces in VGPRs when built with
// the VGPR MFMA form, which a long-lived accumulator does not need: this
// form leaves the 256 VGPRs to operands and softmax temporaries. The
// statement carries its own hazard wait (two wait states between a vector
// ALU write of an operand and the MFMA read of it), since the compiler's
// hazard tracking does not look inside asm.
__device__ __forceinline__ void mfma_acc_agpr(f32x16 &acc, bf16x8 a, bf16x8 b)
{
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The same, as a volatile statement: kept in program order with the other
// volatile statements (slot_done below), for hand-scheduled loops.
__device__ __forceinline__ void mfma_acc_agpr_ordered(f32x16 &acc, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The ordered form without a wait of its own, for hand-scheduled loops in
// which every operand's last vector ALU write lies far enough ahead of the
// MFMA anyway: the ISA hazard test checks that in the generated code of
// every kernel, along every path, so a schedule change that brings a write
// too close fails that test instead of reading a stale operand.
__device__ __forceinline__ void mfma_acc_agpr_nowait(f32x16 &acc, bf16x8 a, bf16x8 b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Marks a value as needed at this point of a hand-scheduled loop: code that
// computes it cannot be sunk past the next ordered MFMA.
__device__ __forceinline__ void slot_done(float x)
{
    asm volatile("" ::"v"(x));
}
__device__ __forceinline__ void slot_done(bf16x8 x)
{
    asm volatile("" ::"v"(x));
}

// Uses a register value here, so that the compiler waits for the load that
// produced it here (before a loop) rather than at its first use inside the
// loop, where that wait would also stall on the loop's own prefetches.
__device__ __forceinline__ void wait_loaded(const bf16x8 &x)
{
    asm volatile("" ::"v"(x));
}
__device__ __forceinline__ void wait_loaded(float x)
{
    asm volatile("" ::"v"(x));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 in order: an
// unrolled loop whose index is a compile-time constant in the body, for
// bodies too large for the loop unroller.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Moves a long-lived MFMA operand into AGPRs: the MFMA reads its A and B
// operands from AGPRs as well as VGPRs, so an operand used only by MFMAs
// stays there and leaves the VGPRs to the values the vector ALU works on.
__device__ __forceinline__ void keep_in_agpr(bf16x8 &x)
{
    asm volatile("" : "+a"(x));
}

// Wait states between the last AGPR-accumulating MFMA and any vector
// instruction that reads its accumulator (more than the 8-pass MFMA needs).
__device__ __forceinline__ void mfma_drain()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Re-defines an accumulator in place, after mfma_drain(): copies the compiler
// makes of it (to VGPRs for the epilogue, or at a control-flow join) then read
// this value, which exists only once the wait states have passed, instead of
// the MFMA result the compiler cannot see is still in flight.
__device__ __forceinline__ void mfma_settle(f32x16 &acc)
{
    asm volatile("" : "+a"(acc));
}

// Direct global->LDS loads (each lane's 16 or 4 bytes land at
// lds_block + lane * size, lds_block wave-uniform), issued as asm. The
// compiler's wait-count pass treats its own direct-load builtin as a write
// to all of LDS and waits for it before the next LDS read of any buffer,
// which exposes the full load latency right after a prefetch is issued;
// asm loads are not tracked, so the caller waits (lds_dma_wait) before the
// barrier that hands the filled buffer to the other waves.
//
// Each load is preceded by one wait state (s_nop 0) inside its asm: the LDS
// address comes from M0, which the compiler writes with an SALU move right
// before the asm, and the ISA requires one wait state between an SALU write
// of M0 and a global/buffer load with LDS = 1. The compiler's hazard check
// does not look inside asm; without the wait a load can take the previous
// M0 and fill the previous 1 KB block, leaving its own block stale.
__device__ __forceinline__ uint32_t lds_byte_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void lds_dma_b128(const void *gsrc, uint32_t lds_block)
{
    asm volatile("s_nop 0\n\t" "global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_block))
                 : "memory");
}
__device__ __forceinline__ void lds_dma_b32(const void *gsrc, uint32_t lds_block)
{
    asm volatile("s_nop 0\n\t" "global_load_lds_dword %0, off" ::"v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_block))
                 : "memory");
}
// The same with a wave-uniform base (SGPR pair) and a 32-bit per-lane byte
// offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_dma_b128_at(const void *gbase, uint32_t off, uint32_t lds_block)
{
    asm volatile("s_nop 0\n\t" "global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(gbase),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_block))
                 : "memory");
}
__device__ __forceinline__ void lds_dma_b32_at(const void *gbase, uint32_t off, uint32_t lds_block)
{
    asm volatile("s_nop 0\n\t" "global_load_lds_dword %0, %1" ::"v"(off), "s"(gbase),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_block))
                 : "memory");
}
// Buffer resource for `bytes` bytes from `base` (raw, stride 0): a buffer
// load at or past the end returns zeros instead of touching memory, which
// lets a tile that runs past the last row be loaded without clamping.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
// Buffer direct loads into LDS (same LDS placement as above); `off` is the
// per-lane byte offset into the resource.
__device__ __forceinline__ void lds_dma_buf_b128(i32x4 rsrc, uint32_t off, uint32_t lds_block)
{
    asm volatile("s_nop 0\n\t" "buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_block))
                 : "memory");
}
__device__ __forceinline__ void lds_dma_buf_b32(i32x4 rsrc, uint32_t off, uint32_t lds_block)
{
    asm volatile("s_nop 0\n\t" "buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_block))
                 : "memory");
}
// An address the compiler must treat as opaque: it keeps one register for it
// and folds the constants added to it into the LDS instruction's offset
// field instead of re-deriving an address per read.
__device__ __forceinline__ uint32_t opaque_addr(uint32_t x)
{
    asm("" : "+v"(x));
    return x;
}
// Workgroup barrier that waits for none of this wave's own LDS reads: a
// caller reading, across it, data that no wave writes until a later barrier
// keeps those reads in flight. Memory accesses are not moved across it.
__device__ __forceinline__ void barrier_reads_in_flight()
{
    asm volatile("s_barrier" ::: "memory");
}

// Waits until every LDS read this wave has issued has returned; memory
// accesses are not moved across it.
__device__ __forceinline__ void lds_reads_wait_all()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products of
// counter words 0 and 2 with 0xD2511F53 and 0xCD9E8D57, the new counter being
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)), the key
// advanced by (0x9E3779B9, 0xBB67AE85) between rounds.
struct Philox4 {
    uint32_t w[4];
};
// 32 x 32 -> 64-bit product in one v_mad_u64_u32 (the compiler otherwise
// spends a v_mul_hi_u32 and a v_mul_lo_u32 on it); m is wave-uniform.
__device__ __forceinline__ uint64_t mul_wide_u32(uint32_t a, uint32_t m)
{
    uint64_t r, carry;
    asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(r), "=s"(carry) : "v"(a), "s"(m));
    return r;
}
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = mul_wide_u32(c0, 0xD2511F53u);
        const uint64_t p1 = mul_wide_u32(c2, 0xCD9E8D57u);
        c0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        c1 = (uint32_t)p1;
        c2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c3 = (uint32_t)p0;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// Dropout parameters: element (i, j) of head bh is kept iff word j % 4 of
// Philox4x32-10(counter (j / 4, i, bh, 0), key (seed_lo, seed_hi)) is at
// least `threshold` (floor(p 2^32)); kept weights are scaled by inv_keep.
struct DropParams {
    uint32_t threshold;
    uint32_t seed_lo, seed_hi;
    float inv_keep;
};
// Keep bits of the 4 consecutive keys j0..j0+3 (j0 % 4 == 0) of query i.
__device__ __forceinline__ uint32_t drop_keep4(const DropParams &dp, uint32_t j0, uint32_t i,
                                               uint32_t bh)
{
    const Philox4 r = philox4x32_10(j0 / 4, i, bh, 0u, dp.seed_lo, dp.seed_hi);
    return (uint32_t)(r.w[0] >= dp.threshold) | ((uint32_t)(r.w[1] >= dp.threshold) << 1) |
           ((uint32_t)(r.w[2] >= dp.threshold) << 2) | ((uint32_t)(r.w[3] >= dp.threshold) << 3);
}

// A buffer offset past the end of every resource used here (tensor slabs are
// below 2^31 bytes): a load from it returns zeros. Used for the columns of a
// padded head dimension.
constexpr uint32_t kBufferOutOfRange = 0x80000000u;

// Waits until at most N of this wave's vector memory operations (the
// direct loads included) are outstanding.
template <int N>
__device__ __forceinline__ void lds_dma_wait()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Eight consecutive bf16 values from LDS (16-byte aligned address).
__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

// Reads at LDS byte addresses (a constant part of the address is folded into
// the instruction's offset field).
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
__device__ __forceinline__ bf16x8 lds_b128_at(uint32_t a)
{
    return *(const lds_bf16x8 *)(size_t)a;
}
__device__ __forceinline__ f32x4 lds_f32x4_at(uint32_t a)
{
    return *(const lds_f32x4 *)(size_t)a;
}
__device__ __forceinline__ bf16x8 lds_tr_pair_at(uint32_t a0, uint32_t a1)
{
    s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(size_t)a0);
    s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(size_t)a1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, ab);
}

// Two transpose reads (4 + 4 values) forming one 8-slot MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint16_t *p0, const uint16_t *p1)
{
    s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0));
    s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p1));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, ab);
}

// Registers 8h..8h+7 of an fp32 accumulator tile, rounded to bf16 (RNE).
__device__ __forceinline__ bf16x8 pack_bf16x8(const f32x16 &c, int h)
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = (__bf16)c[8 * h + i];
    return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float exp2_fast(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

// Each lane gets {x, x of the lane 32 away} from one v_permlane32_swap (the
// upper half of the first copy trades places with the lower half of the
// second), so the reduction over the two halves is one VALU op more and
// stays out of the LDS queue.
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float y;
    asm("v_max_f32 %0, %1, %2" : "=v"(y) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return y;
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait states between an MFMA's write of an accumulator and the first read of
// it by inline asm (the row maxima below read freshly computed scores): the
// ISA requires 12 after v_mfma_f32_32x32x16_bf16 (20 after the fp8
// v_mfma_scale_f32_32x32x64_f8f6f4) before a vector ALU instruction reads the
// result. The compiler inserts them before its own instructions but does not
// look inside asm, so an asm reader it places right behind the MFMA would
// read the registers' previous contents. An asm chain that starts at one
// register of an accumulator therefore first passes that register through a
// compiler-visible add of +0 (not an identity for -0, so it is kept): the
// compiler inserts before it just the wait states its own schedule still
// needs, the chain's first asm reads its result, and every register of the
// accumulator is written by then.
__device__ __forceinline__ void mfma_result_touch(f32x16 &x, int i)
{
    x[i] += 0.f;
}

// Max of three scores without the NaN-quieting copies fmaxf brings in IEEE
// mode (no operand here is ever NaN; -inf is an ordinary value). An operand
// fresh from an MFMA must have passed mfma_result_touch first.
__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    float y;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(y) : "v"(a), "v"(b), "v"(c));
    return y;
}
__device__ __forceinline__ float vmax2(float a, float b)
{
    float y;
    asm("v_max_f32 %0, %1, %2" : "=v"(y) : "v"(a), "v"(b));
    return y;
}

// Asks the scheduler to interleave, within the current basic block, NM
// groups of {1 MFMA, DSR LDS reads, NV vector ALU ops}, so that the vector
// work of a wave issues in the shadow of its own matrix instructions.
template <int NM, int DSR, int NV>
__device__ __forceinline__ void sched_interleave()
{
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        if (DSR > 0)
            __builtin_amdgcn_sched_group_barrier(0x100, DSR, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);       // VALU
    }
}

// Walks the kept blocks of one row (or column) of the block mask in order,
// 64 blocks at a time: each lane of the wave reads one entry of a 64-block
// window (entries `stride` bytes apart), one ballot turns the window into a
// keep bitmask, and the next kept block is the lowest set bit at or after the
// asked position. A window is read again only when the walk leaves it, so a
// row of nb blocks costs ceil(nb / 64) parallel loads instead of one
// dependent load per tile. The whole wave must call it with the same
// arguments (the ballot needs every lane).
struct MaskCursor {
    const uint8_t *base;  // entry j at base[j * stride]
    int stride, nb;
    int w0;               // first block of the window in `bits`
    uint64_t bits;        // keep bits of blocks w0 .. w0 + 63

    __device__ __forceinline__ void init(const uint8_t *base_, int stride_, int nb_)
    {
        base = base_;
        stride = stride_;
        nb = nb_;
        w0 = -(1 << 30);
        bits = 0;
    }
    // Smallest kept block >= j, or nb when there is none.
    __device__ __forceinline__ int next(int j)
    {
        while (j < nb) {
            if (j < w0 || j >= w0 + 64) {
                const int e = j + (int)(threadIdx.x % kWave);
                const bool keep = e < nb && base[(size_t)e * stride] != 0;
                bits = __ballot(keep);
                w0 = j;
            }
            const uint64_t m = bits >> (j - w0);
            if (m != 0)
                return j + __builtin_ctzll(m);
            j = w0 + 64;
        }
        return nb;
    }
};

// First tile at or after t whose mask block is kept (tiles of kMaskBlock /
// tpb rows, tpb tiles per mask block), or `end` when none is left before it.
__device__ __forceinline__ int next_kept_tile(MaskCursor &mc, int t, int end, int tpb)
{
    if (t >= end)
        return end;
    const int b = t / tpb;
    const int kb = mc.next(b);
    if (kb != b)
        t = kb * tpb;
    return t < end ? t : end;
}

// Maps a launched workgroup to a work item so that each XCD (workgroups are
// dealt to the XCDs round-robin) receives one contiguous range of the work
// list: items of one head then run on one XCD and share its L2.
__device__ __forceinline__ int xcd_work_item(int per_xcd)
{
    const int b = blockIdx.x;
    return (b % kXcds) * per_xcd + (b / kXcds);
}

}  // namespace fa
