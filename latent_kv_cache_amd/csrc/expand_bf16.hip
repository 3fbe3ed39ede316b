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
// Tiling.  A block covers 256 output columns of 2048 tokens of one sequence; each of its
// 8 waves owns 32 output columns and keeps their 32 x 512 weight rows in registers as
// two MFMA A operands for the whole block; 64-token latent tiles are staged in LDS
// (32-byte row pad, bank-conflict free) and read as the B operand.
//   out^T[col][token] = W[col][r] . c^T[r][token]
// so lane (q, r16) ends with 4 consecutive columns of token r16: 8-byte stores.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int DH = 128, DR = 64, RK = 512;
constexpr int XT = 64;                  // tokens per tile
constexpr int XSTRIDE = RK + 16;        // LDS row stride of a staged latent tile (8 x odd dwords mod 64)

// Block = 8 waves x 32 output columns (256 columns) x 2048 tokens.  A wave keeps the 32
// weight rows of its columns in registers (two 16-row A operands) for the whole block,
// so each 16-byte latent operand read from LDS feeds two MFMAs; the next 64-token tile
// is loaded into registers while the current one is multiplied.
// One-dimensional, XCD-aware grid: the 2g d_h / 256 column blocks of one token chunk get
// ids 8 apart, so they run on one XCD and all but the first read the chunk's latent
// rows from that XCD's L2 instead of HBM.
constexpr int XCOLS = 256;              // output columns per block
constexpr int XTOK_BLOCK = 2048;        // tokens per block (32 tiles)

template <int G>
__global__ __launch_bounds__(512) void expand_kernel(
    const u16* __restrict__ latent, int64_t lbs, const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int row_begin, int batch, int n_chunks,
    u16* __restrict__ gc, int64_t gbs) {
    constexpr int WOUT = 2 * G * DH + DR;
    constexpr int WIN = RK + DR;
    constexpr int NST = XT * (RK / 8) / 512;   // 16-byte chunks per thread per tile
    __shared__ __attribute__((aligned(16))) u16 lds[2 * XT * XSTRIDE];

    constexpr int NCB = 2 * G * DH / XCOLS;    // column blocks
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int cb = slot % NCB;
    const int chunk = (slot / NCB) * 8 + xcd;
    if (chunk >= n_chunks) return;
    // Chunk-major numbering with the sequence rotated by the chunk index: chunk c of
    // sequence b lands on XCD (b - c) mod 8 (batch a multiple of 8), so ragged lengths,
    // whose late chunks are mostly empty, still spread their work over every XCD.
    const int c = chunk / batch, bb = chunk - c * batch;
    const int b = bb + c % batch < batch ? bb + c % batch : bb + c % batch - batch;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int tbeg = row_begin + c * XTOK_BLOCK;
    if (tbeg >= L) return;
    const int tend = min(tbeg + XTOK_BLOCK, L);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int col0 = cb * XCOLS + wave * 32;   // first output column of this wave
    auto wrow = [&](int col) {
        return col < G * DH ? w_uk + (size_t)col * RK : w_uv + (size_t)(col - G * DH) * RK;
    };
    const u16* w0 = wrow(col0 + r16);
    const u16* w1 = wrow(col0 + 16 + r16);
    bf16x8 wa0[RK / 32], wa1[RK / 32];
#pragma unroll
    for (int ks = 0; ks < RK / 32; ++ks) {
        wa0[ks] = ld_bf16x8(w0 + ks * 32 + q4 * 8);
        wa1[ks] = ld_bf16x8(w1 + ks * 32 + q4 * 8);
    }

    const u16* src = latent + (size_t)b * lbs;
    u16* dst = gc + (size_t)b * gbs;
    // latent rows of a tile: chunk c = k*512 + tid is row c/64, columns 8(c%64)..; rows past
    // the block's end load its last row (in bounds, results not stored)
    u32x4 st[NST];
    auto load_tile = [&](int tb) {
        const int last = tend - 1 - tb;
#pragma unroll
        for (int k = 0; k < NST; ++k) {
            const int c = k * 512 + tid;
            st[k] = *reinterpret_cast<const u32x4*>(src + (size_t)(tb + min(c >> 6, last)) * WIN + (c & 63) * 8);
        }
    };
    // two LDS tiles: the next tile is stored into the other buffer after this one's
    // MFMAs, so one barrier per tile suffices
    auto store_tile = [&](u16* buf) {
#pragma unroll
        for (int k = 0; k < NST; ++k) {
            const int c = k * 512 + tid;
            *reinterpret_cast<u32x4*>(buf + (c >> 6) * XSTRIDE + (c & 63) * 8) = st[k];
        }
    };
    load_tile(tbeg);
    store_tile(lds);
    __syncthreads();
    for (int tb = tbeg, it = 0; tb < tend; tb += XT, ++it) {
        const int nr = min(XT, tend - tb);
        const u16* cur = lds + (it & 1) * (XT * XSTRIDE);
        // the first column block also copies the rotary keys
        if (cb == 0) {
            for (int c = tid; c < nr * (DR / 8); c += 512) {
                const int r = c >> 3, col = c & 7;
                *reinterpret_cast<u32x4*>(dst + (size_t)(tb + r) * WOUT + 2 * G * DH + col * 8) =
                    *reinterpret_cast<const u32x4*>(src + (size_t)(tb + r) * WIN + RK + col * 8);
            }
        }
        if (tb + XT < tend) load_tile(tb + XT);
        // two 16-token tiles at a time: four independent accumulator chains per wave
#pragma unroll
        for (int np = 0; np < XT / 32; ++np) {
            floatx4 acc[2][2] = {};
            const u16* brow = cur + (np * 32 + r16) * XSTRIDE + q4 * 8;
            // operands read three k-steps ahead of their MFMAs (LDS latency)
            constexpr int PF = 3;
            bf16x8 bq[PF][2];
#pragma unroll
            for (int ks = 0; ks < PF; ++ks) {
                bq[ks][0] = ld_bf16x8(brow + ks * 32);
                bq[ks][1] = ld_bf16x8(brow + 16 * XSTRIDE + ks * 32);
            }
#pragma unroll
            for (int ks = 0; ks < RK / 32; ++ks) {
                const bf16x8 b0 = bq[ks % PF][0], b1 = bq[ks % PF][1];
                if (ks + PF < RK / 32) {
                    bq[ks % PF][0] = ld_bf16x8(brow + (ks + PF) * 32);
                    bq[ks % PF][1] = ld_bf16x8(brow + 16 * XSTRIDE + (ks + PF) * 32);
                }
                acc[0][0] = mfma16(wa0[ks], b0, acc[0][0]);
                acc[0][1] = mfma16(wa1[ks], b0, acc[0][1]);
                acc[1][0] = mfma16(wa0[ks], b1, acc[1][0]);
                acc[1][1] = mfma16(wa1[ks], b1, acc[1][1]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tok = np * 32 + h * 16 + r16;
                if (tok < nr) {
                    u16* o = dst + (size_t)(tb + tok) * WOUT + col0 + q4 * 4;
                    *reinterpret_cast<u32x2*>(o) = u32x2{pack2f(acc[h][0][0], acc[h][0][1]), pack2f(acc[h][0][2], acc[h][0][3])};
                    *reinterpret_cast<u32x2*>(o + 16) =
                        u32x2{pack2f(acc[h][1][0], acc[h][1][1]), pack2f(acc[h][1][2], acc[h][1][3])};
                }
            }
        }
        if (tb + XT < tend) store_tile(lds + ((it + 1) & 1) * (XT * XSTRIDE));
        __syncthreads();
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
    const int cps = (span + XTOK_BLOCK - 1) / XTOK_BLOCK;
    const int n_chunks = cps * a.batch;
    dim3 grid(((n_chunks + 7) / 8) * 8 * (2 * G * DH / XCOLS));
    hipLaunchKernelGGL(expand_kernel<G>, grid, dim3(512), 0, st, (const u16*)a.latent, a.latent_bstride,
                       (const u16*)a.w_uk, (const u16*)a.w_uv, a.ctx_lens, a.max_ctx, a.row_begin, a.batch, n_chunks,
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
