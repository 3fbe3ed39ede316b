// Device-side helpers shared by the libgqla kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqla {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf2f(u16 h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

__device__ __forceinline__ uint32_t pack2(u16 lo, u16 hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

__device__ __forceinline__ uint32_t pack2f(float lo, float hi) { return pack2(f2bf(lo), f2bf(hi)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const u16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(u32x4{0u, 0u, 0u, 0u}); }

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies A[m = l%16][k-slot 8*(l/16)+e]
// and B[k-slot 8*(l/16)+e][n = l%16], e = 0..7; D lane l holds D[m = 4*(l/16)+i][n = l%16].
// A and B share the hardware k-slot numbering, so any fixed assignment of contraction
// indices to (l/16, e) that both operands follow gives the same product.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same lane layout with fp16 operands.  The decode kernels keep bf16 in HBM but feed
// the MFMA fp16: its 10-bit mantissa keeps the absorbed query and the softmax weights
// P eight times closer to their fp32 values than bf16 would, at the same MFMA rate.
__device__ __forceinline__ floatx4 mfma16h(f16x8 a, f16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ f16x8 ld_f16x8(const u16* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f16x8 zero_f16x8() { return as_f16x8(u32x4{0u, 0u, 0u, 0u}); }

// Two packed bf16 -> two packed fp16.  Exact for magnitudes in [2^-14, 65504]; smaller
// values lose low bits (fp16 subnormals), larger ones saturate (round toward zero).
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t v) {
    const float lo = __uint_as_float(v << 16);
    const float hi = __uint_as_float(v & 0xffff0000u);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ u32x4 bf8_to_h8(u32x4 v) {
    return u32x4{bf2_to_h2(v[0]), bf2_to_h2(v[1]), bf2_to_h2(v[2]), bf2_to_h2(v[3])};
}

// fp32 -> fp16, round to nearest even.
__device__ __forceinline__ u16 f2h(float f) { return __builtin_bit_cast(u16, (_Float16)f); }

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two packed fp16, round to nearest even (one v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{lo, hi}), halfx2));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16, gfx950).  Every lane addresses 8 bytes
// (4 halfwords).  Within each group of 16 lanes, result lane j, element e is element
// j%4 of what lane 4e + j/4 of the group addressed.  So if the 16 lanes of a group
// address 4 consecutive columns of 4 rows (lane m: row m/4, columns 4(m%4)..+3), lane
// j receives column j of those 4 rows: a 4 x 16 block read as its transpose.
__device__ __forceinline__ u32x2 lds_read_tr16(const u16* p) {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the four lanes l%16 + 16q (q = 0..3) that hold one matrix row, with
// gfx950's cross-row VALU permutes instead of LDS-routed shuffles.  permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of its second;
// permlane32_swap exchanges the upper half of the first with the lower half of the
// second.  Called with the same value twice, the two results hold, in every lane, the
// values of lanes l and l^16 (then l and l^32), one in each result.
__device__ __forceinline__ float wave_max16x4(float v) {
    const uint32_t x = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t y = __float_as_uint(v);
    const auto c = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float wave_sum16x4(float v) {
    const uint32_t x = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t y = __float_as_uint(v);
    const auto c = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---------------------------------------------------------------------------
// Split-K work items.  With the planned chunk c (a multiple of the 32-token tile),
// sequence b of length L gives n = ceil(L / c) items, the chunks whose partials the
// combine merges.  How the n chunks cut the sequence, and the order of the items over
// the grid, depend on whether all items of the launch run at once (at most `cap`
// items, the concurrent workgroups of the device divided by the workgroups per item):
// - One round: the chunks of a sequence are of equal size, cb = ceil(L / n) rounded up
//   to a multiple of 32 (cb <= c, and ceil(L / cb) = n), the last one the rest, in
//   sequence order.  A ragged batch then has no short last chunks: all items are
//   between about c (n - 1) / n and c tokens, and the planner can pick c so that they
//   fill the compute units evenly.
// - Several rounds: chunks of c tokens and a shorter last one; every full chunk first,
//   sequence by sequence, then the last chunks, longest first.  The dispatcher hands
//   blocks to compute units in grid order as they free up, so the long items start
//   first and the short ones fill the last round in.
// Batches above kSortTails sequences keep their last chunks in sequence order.
// chunk_of_item maps item k to (sequence b, chunk p, tokens [t0, t1)); false when k is
// past the last item.  Every thread of the block calls it with the same k.  sh: LDS
// scratch of at least NT / 64 + 2 + 2 min(batch, kSortTails) ints (the tile buffer,
// before its first use).
// ---------------------------------------------------------------------------
constexpr int kSortTails = 1024;
constexpr int kChunkAlign = 32;

__device__ __forceinline__ int chunks_of(int L, int chunk) { return (L + chunk - 1) / chunk; }
__device__ __forceinline__ int chunk_size(int L, int n) {
    return ((L + n - 1) / n + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
}

template <int NT>
__device__ __forceinline__ bool chunk_of_item(int k, const int32_t* __restrict__ ctx_lens, int batch, int max_ctx,
                                              int chunk, int cap, int* sh, int& b_out, int& p_out, int& t0_out,
                                              int& t1_out) {
    constexpr int NWV = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    auto len_of = [&](int b) { return clampi(ctx_lens[b], 0, max_ctx); };
    // Block-wide exclusive scan of v(i) over i < batch: the one thread whose i has v > 0
    // and holds position kk in [excl, excl + v) stores i and kk - excl at sh[NWV],
    // sh[NWV + 1].  Returns the total.
    auto scan_find = [&](auto v_of, int kk) -> int {
        int run = 0;
        for (int base = 0; base < batch; base += NT) {
            const int i = base + tid;
            const int v = i < batch ? v_of(i) : 0;
            int x = v;   // inclusive scan over the wave
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            if (lane == 63) sh[wv] = x;
            __syncthreads();
            int woff = 0, ctot = 0;
#pragma unroll
            for (int w = 0; w < NWV; ++w) {
                woff += w < wv ? sh[w] : 0;
                ctot += sh[w];
            }
            const int excl = run + woff + x - v;
            __syncthreads();
            if (v > 0 && excl <= kk && kk < excl + v) {
                sh[NWV] = i;
                sh[NWV + 1] = kk - excl;
            }
            run += ctot;
        }
        __syncthreads();
        return run;
    };
    const bool sorted = batch <= kSortTails;
    int* key = sh + NWV + 2;   // per sequence: last-chunk length
    int* perm = key + batch;   // sequences by decreasing key, ties in sequence order

    // all items in sequence order; the total decides between one round and several
    const int total = scan_find([&](int b) { return chunks_of(len_of(b), chunk); }, k);
    if (k >= total) return false;   // past the last item
    if (total <= cap) {
        // every item starts at once, so their order does not matter
        const int b = sh[NWV];
        const int p = sh[NWV + 1];
        const int L = len_of(b), cb = chunk_size(L, chunks_of(L, chunk));
        b_out = b;
        p_out = p;
        t0_out = p * cb;
        t1_out = min(t0_out + cb, L);
        return true;
    }
    // full chunks: floor(L_b / c) per sequence
    const int nfull = scan_find([&](int b) { return len_of(b) / chunk; }, k);
    int b, p;
    if (k < nfull) {
        b = sh[NWV];
        p = sh[NWV + 1];
    } else {
        // the (k - nfull)-th last chunk in order of decreasing length
        const int i = k - nfull;
        if (sorted) {
            for (int c = tid; c < batch; c += NT) key[c] = len_of(c) % chunk;
            __syncthreads();
            for (int b = tid; b < batch; b += NT) {
                const int kb = key[b];
                int rank = 0;
                for (int c = 0; c < batch; ++c) {
                    const int kc = key[c];
                    rank += (kc > kb) || (kc == kb && c < b);
                }
                perm[rank] = b;
            }
            __syncthreads();
        }
        scan_find([&](int r) { return len_of(sorted ? perm[r] : r) % chunk ? 1 : 0; }, i);
        b = sorted ? perm[sh[NWV]] : sh[NWV];
        p = len_of(b) / chunk;
    }
    b_out = b;
    p_out = p;
    t0_out = p * chunk;
    t1_out = min(t0_out + chunk, len_of(b));
    return true;
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS byte address lds_base + 16 l; lds_base must be wave-uniform.  It is
// issued from inline assembly so that the compiler, which cannot tell which LDS bytes
// such a load writes, does not wait for all of them before every later LDS access;
// callers wait with wait_vmcnt<> before reading the destination.  The compiler does not
// count these loads, so its own waits on later global loads only over-wait (loads
// retire in issue order).  The global address is a wave-uniform 64-bit base (SGPRs)
// plus a 32-bit per-lane byte offset.  Lanes outside EXEC write nothing.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}

// dma16 with the streaming hint (nt): for data that is read once.
__device__ __forceinline__ void dma16_nt(const void* gbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds_base), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt immediate on gfx9: vmcnt = bits [3:0] and [15:14]; expcnt and
    // lgkmcnt fields left at their maxima (no wait on them)
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier without the compiler's memory fence (whose vmcnt(0) would drain the direct
// loads still in flight): own LDS operations complete, then s_barrier.
__device__ __forceinline__ void block_sync() {
    asm volatile("" ::: "memory");
    // s_waitcnt lgkmcnt(0): vmcnt field at its maximum 63 (bits [3:0] and [15:14]),
    // expcnt at 7, lgkmcnt (bits [11:8]) at 0
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace gqla
