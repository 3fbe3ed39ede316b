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
// two MFMA A operands for the whole block; 32-token latent tiles are staged in LDS
// (32-byte row pad, bank-conflict free) and read as the B operand.
//   out^T[col][token] = W[col][r] . c^T[r][token]
// so lane (q, r16) ends with 4 consecutive columns of token r16; these are staged in LDS
// and leave as 16-byte stores that write whole 512-byte row segments.
#include "common.h"
#include "launch.h"
#include "append_rope.h"

namespace gqla {

namespace {

constexpr int DH = 128, DR = 64, RK = 512;
constexpr int XT = 64;                  // tokens per tile
constexpr int XSTRIDE = RK + 16;        // LDS row stride of a staged latent tile (8 x odd dwords mod 64)

// Block = 8 waves x 32 output columns (256 columns) x 2048 tokens.  A wave keeps the 32
// weight rows of its columns in registers (two 16-row A operands) for the whole block,
// so each 16-byte latent operand read from LDS feeds two MFMAs.
// One-dimensional, XCD-aware grid: the 2g d_h / 256 column blocks of one token chunk get
// ids 8 apart, so they run on one XCD and all but the first read the chunk's latent
// rows from that XCD's L2 instead of HBM.
// Steps of ET tokens over three input and two output LDS buffers.  At step k, after the
// barrier that published input tile k:
//   - the latent rows of tile k+2 go from global memory straight into an input buffer
//     (global_load_lds_dwordx4, one wave instruction per 1 KB row), so every load has
//     two steps to land;
//   - the MFMAs of tile k run, and between them every thread stores two 16-byte pieces
//     of tile k-1's output from output buffer (k-1)%2 (each wave instruction writes two
//     whole 512-byte row segments);
//   - the MFMA results of tile k are written to output buffer k%2;
//   - each wave waits for its loads of tile k+1 (not for anything issued after them),
//     then the barrier.
// The first column block also copies the rotary keys, staged through LDS with the tile.
constexpr int XCOLS = 256;              // output columns per block
constexpr int OSTRIDE = XCOLS + 8;      // LDS row stride of a staged output tile
constexpr int XTOK_BLOCK = 2048;        // tokens per block
constexpr int ET = 32;                  // tokens per step
constexpr int NIB = 3;                  // input buffers
constexpr int EPF = 3;                  // k-steps an LDS operand read runs ahead of its MFMAs
constexpr int EXW = 8;                  // waves per block (32 columns each)

template <int G, int NW>
__global__ __launch_bounds__(NW * 64) void expand_kernel(
    const u16* __restrict__ latent, int64_t lbs, const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int row_begin, int batch, int n_chunks,
    u16* __restrict__ gc, int64_t gbs) {
    constexpr int NT = NW * 64;                  // threads
    constexpr int CT = XCOLS / 16 / NW;          // 16-column MFMA tiles per wave
    constexpr int RPW = ET / NW;                 // latent rows each wave loads per tile
    constexpr int RLN = ET * (DR / 8) / NW;      // lanes per wave that load / store rotary keys
    constexpr int EST = ET * (XCOLS / 8) / NT;   // 16-byte output stores per thread per step
    constexpr int KS = RK / 32;                  // k-steps
    static_assert(RLN <= 64 && RPW * NW == ET && EST * NT == ET * (XCOLS / 8), "tile shape");
    constexpr int WOUT = 2 * G * DH + DR;
    constexpr int WIN = RK + DR;
    constexpr int ITILE = ET * XSTRIDE, RTILE = ET * DR, OTILE = ET * OSTRIDE;   // u16 elements
    __shared__ __attribute__((aligned(16))) u16 lds[NIB * (ITILE + RTILE) + 2 * OTILE];
    auto ibuf = [&](int i) -> u16* { return lds + i * ITILE; };
    auto rbuf = [&](int i) -> u16* { return lds + NIB * ITILE + i * RTILE; };
    auto obuf = [&](int k) -> u16* { return lds + NIB * (ITILE + RTILE) + (k & 1) * OTILE; };

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
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q4 = lane >> 4, r16 = lane & 15;
    const bool rope = cb == 0;
    const int col0 = cb * XCOLS + wave * CT * 16;   // first output column of this wave
    bf16x8 wa[CT][KS];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int col = col0 + ct * 16 + r16;
        const u16* w = col < G * DH ? w_uk + (size_t)col * RK : w_uv + (size_t)(col - G * DH) * RK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) wa[ct][ks] = ld_bf16x8(w + ks * 32 + q4 * 8);
    }

    const u16* src = latent + (size_t)b * lbs;
    u16* dst = gc + (size_t)b * gbs;
    // Tile tb into input buffer i: wave w loads rows w, w + NW, ..; rows past the block's
    // end load its last row (in bounds, results not stored).  With the rotary keys, lanes
    // 0..RLN-1 of wave w also load those of rows w RLN / 8 .. into the tile's rope area.
    // Loads per wave: RPW, plus one with the rotary keys.
    const int rr = wave * (RLN / 8) + (lane >> 3), rc = (lane & 7) * 8;   // rotary row and column
    auto load_tile = [&](int tb, int i) {
        const int last = tend - 1 - tb;
        const uint32_t lb = lds_addr(ibuf(i));
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int r = k * NW + wave;
            dma16(src + (size_t)(tb + min(r, last)) * WIN, (uint32_t)lane * 16u, lb + (uint32_t)(r * XSTRIDE * 2));
        }
        if (rope && lane < RLN)
            dma16(src + (size_t)tb * WIN + RK, (uint32_t)(min(rr, last) * WIN + rc) * 2u,
                  lds_addr(rbuf(i) + wave * (RLN / 8) * DR));
    };
    // Piece j (< EST) of this thread's share of a staged output tile: row r, 8 columns.
    // Read from LDS well before the store, so that the store does not wait for every LDS
    // read in flight (LDS operations complete in order).
    auto piece_row = [&](int j) { return (j * NT + tid) / (XCOLS / 8); };
    auto piece_col = [&](int j) { return ((j * NT + tid) % (XCOLS / 8)) * 8; };
    auto read_piece = [&](const u16* ob, int j) {
        return *reinterpret_cast<const u32x4*>(ob + piece_row(j) * OSTRIDE + piece_col(j));
    };
    auto store_piece = [&](u32x4 v, int tb, int nr, int j) {
        const int r = piece_row(j);
        if (r < nr)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + (size_t)(tb + r) * WOUT + cb * XCOLS + piece_col(j)));
    };
    const int ntiles = (tend - tbeg + ET - 1) / ET;
    load_tile(tbeg, 0);
    if (ntiles > 1) load_tile(tbeg + ET, 1);
    // the compiler does not count the direct loads, and a workgroup barrier does not wait
    // for vector memory: each wave waits for its own loads, then the barrier
    wait_vmcnt<0>();
    block_sync();
    int ptb = 0, pnr = 0;   // the previous tile, whose output is stored during this step
    for (int it = 0, bi = 0; it < ntiles; ++it, bi = bi == NIB - 1 ? 0 : bi + 1) {
        const int tb = tbeg + it * ET, nr = min(ET, tend - tb);
        const bool more2 = it + 2 < ntiles;
        // tile it+2 into the buffer that tile it-1 used
        if (more2) load_tile(tb + 2 * ET, bi == 0 ? NIB - 1 : bi - 1);
        const u16* cur = ibuf(bi);
        // tile it-1's output, staged in output buffer (it-1)%2, and this tile's rotary keys
        u32x4 pv[EST], rv;
        if (it > 0) {
#pragma unroll
            for (int j = 0; j < EST; ++j) pv[j] = read_piece(obuf(it + 1), j);
        }
        if (rope && lane < RLN) rv = *reinterpret_cast<const u32x4*>(rbuf(bi) + rr * DR + rc);
        // two 16-token halves: 2 CT independent accumulator chains per wave
        floatx4 acc[2][CT] = {};
        const u16* brow = cur + r16 * XSTRIDE + q4 * 8;
        bf16x8 bq[EPF][2];
#pragma unroll
        for (int ks = 0; ks < EPF; ++ks) {
            bq[ks][0] = ld_bf16x8(brow + ks * 32);
            bq[ks][1] = ld_bf16x8(brow + 16 * XSTRIDE + ks * 32);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 b0 = bq[ks % EPF][0], b1 = bq[ks % EPF][1];
            if (ks + EPF < KS) {
                bq[ks % EPF][0] = ld_bf16x8(brow + (ks + EPF) * 32);
                bq[ks % EPF][1] = ld_bf16x8(brow + 16 * XSTRIDE + (ks + EPF) * 32);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                acc[0][ct] = mfma16(wa[ct][ks], b0, acc[0][ct]);
                acc[1][ct] = mfma16(wa[ct][ks], b1, acc[1][ct]);
            }
            if (it > 0 && ks % (KS / EST) == KS / EST / 2) store_piece(pv[ks / (KS / EST)], ptb, pnr, ks / (KS / EST));
            if (ks == 1 && rope && lane < RLN && rr < nr)   // one rotary store per wave
                __builtin_nontemporal_store(rv, reinterpret_cast<u32x4*>(dst + (size_t)(tb + rr) * WOUT + 2 * G * DH + rc));
            // keeps each k-step's reads EPF steps ahead of their MFMAs (left to itself the
            // scheduler moves every read next to its MFMAs)
            __builtin_amdgcn_sched_barrier(0);
        }
        // this tile's results into output buffer it%2 (its previous contents, tile it-2,
        // were stored during step it-1)
        u16* const ob = obuf(it);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                *reinterpret_cast<u32x2*>(ob + (h * 16 + r16) * OSTRIDE + wave * CT * 16 + ct * 16 + q4 * 4) =
                    u32x2{pack2f(acc[h][ct][0], acc[h][ct][1]), pack2f(acc[h][ct][2], acc[h][ct][3])};
        ptb = tb;
        pnr = nr;
        // This wave's loads of tile it+1 have landed.  Vector memory operations complete
        // in issue order.  Issued after those loads (at the start of step it-1, before
        // the loop for it = 0), and left in flight, are: the stores of step it-1 (EST
        // from step 2 on, and the rope store), the loads of tile it+2 (RPW, and the
        // rope load), and the stores of this step (likewise).  Every tile stored here is
        // full, so no store is skipped; the last tile needs no wait.  Rope blocks
        // over-wait where the counts below leave out their rope operations.
        if (it + 1 < ntiles) {
            if (it == 0)
                wait_vmcnt<0>();
            else if (it == 1)
                more2 ? wait_vmcnt<EST + RPW>() : wait_vmcnt<EST>();
            else if (!more2)
                wait_vmcnt<2 * EST>();
            else if (rope)
                wait_vmcnt<2 * (EST + 1) + RPW + 1>();
            else
                wait_vmcnt<2 * EST + RPW>();
        }
        block_sync();   // every wave's have, tile it is read and its output staged
    }
    // the last tile's output
#pragma unroll
    for (int j = 0; j < EST; ++j) store_piece(read_piece(obuf(ntiles - 1), j), ptb, pnr, j);
}

// Expansion of the decode step's new rows (the append): row r < batch * s_q of c_new
// ([batch][s_q][r_kv], packed) is token s = r % s_q of sequence b = r / s_q, which sits
// at t = L_b - s_q + s of the group cache (rows with t < 0 are skipped).  Same tiling
// as expand_kernel with one 64-row tile per block of NT threads (bx: NT / 4 output
// columns, 16 per wave; by: 64 rows); the rotary key columns are written by the
// append's rotation.
template <int G, int NT>
__device__ __forceinline__ void append_expand_block(
    int bx, int by, const u16* __restrict__ c_new, const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
    const int32_t* __restrict__ ctx_lens, int max_ctx, int s_q, int rows, u16* __restrict__ gc, int64_t gbs) {
    constexpr int WOUT = 2 * G * DH + DR;
    __shared__ __attribute__((aligned(16))) u16 lds[XT * XSTRIDE];

    const int r0 = by * XT;
    const int nr = min(XT, rows - r0);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int col0 = bx * (NT / 4) + wave * 16;
    const int colA = col0 + r16;
    const u16* wrow = colA < G * DH ? w_uk + (size_t)colA * RK : w_uv + (size_t)(colA - G * DH) * RK;

    bf16x8 wa[RK / 32];
#pragma unroll
    for (int ks = 0; ks < RK / 32; ++ks) wa[ks] = ld_bf16x8(wrow + ks * 32 + q4 * 8);
    {
        u32x4 v[XT * (RK / 8) / NT];
#pragma unroll
        for (int k = 0; k < XT * (RK / 8) / NT; ++k) {
            const int c = k * NT + tid;
            const int r = c >> 6, col = c & 63;
            v[k] = u32x4{0u, 0u, 0u, 0u};
            if (r < nr) v[k] = *reinterpret_cast<const u32x4*>(c_new + (size_t)(r0 + r) * RK + col * 8);
        }
#pragma unroll
        for (int k = 0; k < XT * (RK / 8) / NT; ++k) {
            const int c = k * NT + tid;
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

// The whole bf16 append in one launch: blocks below nexp expand the new rows (block i:
// columns bx = i % (2 g d_h / 64), rows by = i / that), the rest rotate one new token
// each.  The two parts touch disjoint outputs and read only inputs, so they run side by
// side instead of one launch after the other.  256 threads: at 512 the expansion's
// weights, operands and accumulators do not fit the registers of two waves per SIMD.
constexpr int APT = 256;
template <int G>
__global__ __launch_bounds__(APT) void append_fused_kernel(
    const u16* __restrict__ c_new, const u16* __restrict__ kr_new, const u16* __restrict__ q_raw,
    u16* __restrict__ q_out, const int32_t* __restrict__ ctx_lens, int max_ctx, int s_q, int h_q, int rows,
    double theta, u16* __restrict__ latent, int64_t lbs, const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
    u16* __restrict__ gc, int64_t gbs, int nexp) {
    constexpr int NCB = 2 * G * DH / (APT / 4);
    const int i = blockIdx.x;
    if (i < nexp)
        append_expand_block<G, APT>(i % NCB, i / NCB, c_new, w_uk, w_uv, ctx_lens, max_ctx, s_q, rows, gc, gbs);
    else
        append_rope_token<u16, APT>(i - nexp, c_new, kr_new, q_raw, q_out, ctx_lens, max_ctx, s_q, h_q, RK, DR, theta,
                                    latent, lbs, gc, gbs, 2 * G * DH);
}

template <int G>
hipError_t launch_append_fused_g(const AppendArgs& a, hipStream_t st) {
    const int rows = a.batch * a.s_q;
    const int nexp = (2 * G * DH / (APT / 4)) * ((rows + XT - 1) / XT);
    hipLaunchKernelGGL(append_fused_kernel<G>, dim3(nexp + rows), dim3(APT), 0, st, (const u16*)a.c_new,
                       (const u16*)a.kr_new, (const u16*)a.q_rope_raw, (u16*)a.q_rope_out, a.ctx_lens, a.max_ctx,
                       a.s_q, a.h_q, rows, (double)a.theta, (u16*)a.latent, a.latent_bstride, (const u16*)a.w_uk,
                       (const u16*)a.w_uv, (u16*)a.group_cache, a.group_bstride, nexp);
    return hipGetLastError();
}

template <int G>
hipError_t launch_expand_g(const ExpandArgs& a, hipStream_t st) {
    const int span = a.max_ctx - a.row_begin;
    if (span <= 0 || a.batch == 0) return hipSuccess;
    const int cps = (span + XTOK_BLOCK - 1) / XTOK_BLOCK;
    const int n_chunks = cps * a.batch;
    dim3 grid(((n_chunks + 7) / 8) * 8 * (2 * G * DH / XCOLS));
    hipLaunchKernelGGL((expand_kernel<G, EXW>), grid, dim3(EXW * 64), 0, st, (const u16*)a.latent, a.latent_bstride,
                       (const u16*)a.w_uk, (const u16*)a.w_uv, a.ctx_lens, a.max_ctx, a.row_begin, a.batch, n_chunks,
                       (u16*)a.group_cache, a.group_bstride);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append_fused_bf16(const AppendArgs& a, hipStream_t st) {
    if (a.batch * a.s_q == 0) return hipSuccess;
    switch (a.g) {
        case 1: return launch_append_fused_g<1>(a, st);
        case 2: return launch_append_fused_g<2>(a, st);
        case 4: return launch_append_fused_g<4>(a, st);
        case 8: return launch_append_fused_g<8>(a, st);
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
