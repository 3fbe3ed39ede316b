// bf16 MFMA group expansion for gfx950.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture, GQA path): the latent
// is expanded into g groups of keys and values once, so that decode does not
// expand it again at every step.  Row t of sequence b becomes
//   [W_UK[0] c_t .. W_UK[g-1] c_t | W_UV[0] c_t .. W_UV[g-1] c_t | k_R,t],
// a GEMM of the latent rows against the stacked up-projections [W_UK; W_UV]
// (2 g d_h rows of width r_kv) plus a copy of the rotary key.
//
// Tiling.  grid = (2g d_h / 128 column blocks, token chunks, batch).  Each of the
// 8 waves of a block owns 16 output columns and keeps their 16 x 512 weight rows
// in registers as the MFMA A operand for the whole chunk; 64-token latent tiles
// are staged in LDS (32-byte row pad, bank-conflict free) and read as the B operand.
//   out^T[col][token] = W[col][r] . c^T[r][token]
// so lane (q, r16) ends with 4 consecutive columns of token r16: one 8-byte store.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int DH = 128, DR = 64, RK = 512;
constexpr int XT = 64;                  // tokens per tile
constexpr int XSTRIDE = RK + 16;        // LDS row stride of a staged latent tile (8 x odd dwords mod 64)
constexpr int XTOK_PER_BLOCK = 256;     // tokens per block (4 tiles)

template <int G>
__global__ __launch_bounds__(512) void expand_kernel(
    const u16* __restrict__ latent, int64_t lbs, const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int row_begin, u16* __restrict__ gc, int64_t gbs) {
    constexpr int WOUT = 2 * G * DH + DR;
    constexpr int WIN = RK + DR;
    __shared__ __attribute__((aligned(16))) u16 lds[XT * XSTRIDE];

    const int b = blockIdx.z;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int tbeg = row_begin + blockIdx.y * XTOK_PER_BLOCK;
    if (tbeg >= L) return;
    const int tend = min(tbeg + XTOK_PER_BLOCK, L);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int col0 = blockIdx.x * 128 + wave * 16;   // first output column of this wave
    const int colA = col0 + r16;                       // weight row this lane supplies
    const u16* wrow = colA < G * DH ? w_uk + (size_t)colA * RK : w_uv + (size_t)(colA - G * DH) * RK;

    bf16x8 wa[RK / 32];
#pragma unroll
    for (int ks = 0; ks < RK / 32; ++ks) wa[ks] = ld_bf16x8(wrow + ks * 32 + q4 * 8);

    const u16* src = latent + (size_t)b * lbs;
    u16* dst = gc + (size_t)b * gbs;

    for (int tb = tbeg; tb < tend; tb += XT) {
        const int nr = min(XT, tend - tb);
        __syncthreads();
        // stage c rows (first 512 columns of each latent row): 8 chunks of 16 bytes per
        // thread, all loads issued before the stores
        {
            u32x4 v[XT * (RK / 8) / 512];
#pragma unroll
            for (int k = 0; k < XT * (RK / 8) / 512; ++k) {
                const int c = k * 512 + tid;
                const int r = c >> 6, col = c & 63;
                v[k] = u32x4{0u, 0u, 0u, 0u};
                if (r < nr) v[k] = *reinterpret_cast<const u32x4*>(src + (size_t)(tb + r) * WIN + col * 8);
            }
#pragma unroll
            for (int k = 0; k < XT * (RK / 8) / 512; ++k) {
                const int c = k * 512 + tid;
                *reinterpret_cast<u32x4*>(lds + (c >> 6) * XSTRIDE + (c & 63) * 8) = v[k];
            }
        }
        // the first column block also copies the rotary keys
        if (blockIdx.x == 0) {
            for (int c = tid; c < nr * (DR / 8); c += 512) {
                const int r = c >> 3, col = c & 7;
                *reinterpret_cast<u32x4*>(dst + (size_t)(tb + r) * WOUT + 2 * G * DH + col * 8) =
                    *reinterpret_cast<const u32x4*>(src + (size_t)(tb + r) * WIN + RK + col * 8);
            }
        }
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < XT / 16; ++nt) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            const u16* brow = lds + (nt * 16 + r16) * XSTRIDE + q4 * 8;
#pragma unroll
            for (int ks = 0; ks < RK / 32; ++ks) acc = mfma16(wa[ks], ld_bf16x8(brow + ks * 32), acc);
            const int tok = nt * 16 + r16;
            if (tok < nr) {
                u32x2 o;
                o[0] = pack2f(acc[0], acc[1]);
                o[1] = pack2f(acc[2], acc[3]);
                *reinterpret_cast<u32x2*>(dst + (size_t)(tb + tok) * WOUT + col0 + q4 * 4) = o;
            }
        }
    }
}

// Expansion of the decode step's new rows (the append): row r < batch * s_q of c_new
// ([batch][s_q][r_kv], packed) is token s = r % s_q of sequence b = r / s_q, which sits
// at t = L_b - s_q + s of the group cache (rows with t < 0 are skipped).  Same tiling
// as expand_kernel with one 64-row tile per block; the rotary key columns are written
// by the append's rotation kernel.
template <int G>
__global__ __launch_bounds__(512) void append_expand_kernel(
    const u16* __restrict__ c_new, const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int s_q, int rows, u16* __restrict__ gc, int64_t gbs) {
    constexpr int WOUT = 2 * G * DH + DR;
    __shared__ __attribute__((aligned(16))) u16 lds[XT * XSTRIDE];

    const int r0 = blockIdx.y * XT;
    const int nr = min(XT, rows - r0);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int col0 = blockIdx.x * 128 + wave * 16;
    const int colA = col0 + r16;
    const u16* wrow = colA < G * DH ? w_uk + (size_t)colA * RK : w_uv + (size_t)(colA - G * DH) * RK;

    bf16x8 wa[RK / 32];
#pragma unroll
    for (int ks = 0; ks < RK / 32; ++ks) wa[ks] = ld_bf16x8(wrow + ks * 32 + q4 * 8);
    {
        u32x4 v[XT * (RK / 8) / 512];
#pragma unroll
        for (int k = 0; k < XT * (RK / 8) / 512; ++k) {
            const int c = k * 512 + tid;
            const int r = c >> 6, col = c & 63;
            v[k] = u32x4{0u, 0u, 0u, 0u};
            if (r < nr) v[k] = *reinterpret_cast<const u32x4*>(c_new + (size_t)(r0 + r) * RK + col * 8);
        }
#pragma unroll
        for (int k = 0; k < XT * (RK / 8) / 512; ++k) {
            const int c = k * 512 + tid;
            *reinterpret_cast<u32x4*>(lds + (c >> 6) * XSTRIDE + (c & 63) * 8) = v[k];
        }
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < XT / 16; ++nt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const u16* brow = lds + (nt * 16 + r16) * XSTRIDE + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < RK / 32; ++ks) acc = mfma16(wa[ks], ld_bf16x8(brow + ks * 32), acc);
        const int r = nt * 16 + r16;
        if (r < nr) {
            const int row = r0 + r;
            const int b = row / s_q, s = row - (row / s_q) * s_q;
            const int t = clampi(ctx_lens[b], 0, max_ctx) - s_q + s;
            if (t >= 0) {
                u32x2 o;
                o[0] = pack2f(acc[0], acc[1]);
                o[1] = pack2f(acc[2], acc[3]);
                *reinterpret_cast<u32x2*>(gc + (size_t)b * gbs + (size_t)t * WOUT + col0 + q4 * 4) = o;
            }
        }
    }
}

template <int G>
hipError_t launch_append_expand_g(const AppendArgs& a, hipStream_t st) {
    const int rows = a.batch * a.s_q;
    dim3 grid(2 * G * DH / 128, (rows + XT - 1) / XT);
    hipLaunchKernelGGL(append_expand_kernel<G>, grid, dim3(512), 0, st, (const u16*)a.c_new, (const u16*)a.w_uk,
                       (const u16*)a.w_uv, a.ctx_lens, a.max_ctx, a.s_q, rows, (u16*)a.group_cache, a.group_bstride);
    return hipGetLastError();
}

template <int G>
hipError_t launch_expand_g(const ExpandArgs& a, hipStream_t st) {
    const int span = a.max_ctx - a.row_begin;
    if (span <= 0 || a.batch == 0) return hipSuccess;
    dim3 grid(2 * G * DH / 128, (span + XTOK_PER_BLOCK - 1) / XTOK_PER_BLOCK, a.batch);
    hipLaunchKernelGGL(expand_kernel<G>, grid, dim3(512), 0, st, (const u16*)a.latent, a.latent_bstride,
                       (const u16*)a.w_uk, (const u16*)a.w_uv, a.ctx_lens, a.max_ctx, a.row_begin,
                       (u16*)a.group_cache, a.group_bstride);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append_expand_bf16(const AppendArgs& a, hipStream_t st) {
    switch (a.g) {
        case 1: return launch_append_expand_g<1>(a, st);
        case 2: return launch_append_expand_g<2>(a, st);
        case 4: return launch_append_expand_g<4>(a, st);
        case 8: return launch_append_expand_g<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_expand_bf16(const ExpandArgs& a, hipStream_t st) {
    switch (a.g) {
        case 1: return launch_expand_g<1>(a, st);
        case 2: return launch_expand_g<2>(a, st);
        case 4: return launch_expand_g<4>(a, st);
        case 8: return launch_expand_g<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gqla
