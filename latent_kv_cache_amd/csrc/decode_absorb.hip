// bf16 MFMA absorb decode for gfx950: the absorbed-query prologue and the latent
// attention kernel with the W_UV up-projection fused into its epilogue.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Architecture, MQA-absorb path).  Head i
// of group j = i / (h_q/g) attends over the shared latent rows [c_t | k_R,t]:
//   q~ = W_UK[j]^T q^N,  score_t = scale [q~ | q^R].[c_t | k_R,t],
//   u = sum_t softmax(score)_t c_t,  o = W_UV[j] u,
// over the visible tokens t <= L_b - s_q + s of query token s, one context chunk per
// workgroup (split-K); each workgroup writes the chunk's o and log-sum-exp and
// launch_combine merges the chunks.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

constexpr int DH = 128;   // per-group value width
constexpr int DR = 64;    // rotary key width
constexpr int RK = 512;   // latent width
constexpr int W = RK + DR;
constexpr int TT = 32;    // tokens per tile

// ---------------------------------------------------------------------------
// Prologue: qhat[b][rho][0:512] = W_UK[j]^T q^N * scale * log2(e) and
// qhat[b][rho][512:576] = q^R * scale * log2(e), rho = s*h_q + h, stored as fp16 (the
// operand type of the attention kernel's MFMA).  With the softmax scale and the
// change of base folded into the query, the attention kernel's scores come out as
// log2-domain logits and need no multiply.
// grid = (row blocks of 64, g, 4 quarters of the latent columns); block = 4 waves.
// Rows of group j are numbered iota = (b*s_q + s)*hpg + hh.  The block's quarter of
// W_UK[j] ([d][r], 128 x 128, 32 KB) is staged row-major in LDS, so four blocks fit on
// a CU; the contraction runs over d, so the A operand (W_UK^T) is formed with
// transposing LDS reads: 4 rows d x 16 columns r per 16-lane group.  The blocks of the
// first quarter also write the scaled q^R.
// ---------------------------------------------------------------------------
constexpr int PRO_COLS = RK / 4;
constexpr int PRO_STRIDE = PRO_COLS + 16;

__global__ __launch_bounds__(256) void absorb_prologue_kernel(
    const u16* __restrict__ q_nope, const u16* __restrict__ q_rope, const u16* __restrict__ w_uk,
    u16* __restrict__ qhat, int batch, int h_q, int g, int s_q, float scale_log2) {
    __shared__ __attribute__((aligned(16))) u16 wt[DH * PRO_STRIDE];
    const int j = blockIdx.y;
    const int r0 = blockIdx.z * PRO_COLS;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;

    // stage columns r0 .. r0+127 of W_UK[j]: 2048 chunks of 16 bytes, 8 per thread, all
    // eight loads in flight before the first store
    const u16* wj = w_uk + (size_t)j * DH * RK + r0;
    constexpr int CPRW = PRO_COLS / 8;   // 16-byte chunks per staged row
    {
        u32x4 v[DH * CPRW / 256];
#pragma unroll
        for (int k = 0; k < DH * CPRW / 256; ++k) {
            const int c = k * 256 + tid;
            v[k] = *reinterpret_cast<const u32x4*>(wj + (size_t)(c / CPRW) * RK + (c % CPRW) * 8);
        }
#pragma unroll
        for (int k = 0; k < DH * CPRW / 256; ++k) {
            const int c = k * 256 + tid;
            *reinterpret_cast<u32x4*>(wt + (c / CPRW) * PRO_STRIDE + (c % CPRW) * 8) = v[k];
        }
    }
    __syncthreads();

    const int hpg = h_q / g;
    const int nrows = batch * s_q * hpg;
    const int iota = blockIdx.x * 64 + wave * 16 + r16;
    const bool ok = iota < nrows;
    const int bs = ok ? iota / hpg : 0;
    const int hh = ok ? iota - bs * hpg : 0;
    const int b = bs / s_q, s = bs - (bs / s_q) * s_q;
    const int h = j * hpg + hh;
    const size_t qrow = ((size_t)b * s_q + s) * h_q + h;
    const int RQ = s_q * h_q;
    u16* dst = qhat + ((size_t)b * RQ + (size_t)s * h_q + h) * W;

    // k-slot e of lane group q4 in k-step kd is d = 32kd + 4q4 + e (e < 4) or
    // 32kd + 16 + 4q4 + (e - 4): the transposing reads of the four lane groups then lie
    // 4 rows apart, 32 banks at this row stride, so they do not conflict
    bf16x8 qb[DH / 32];
#pragma unroll
    for (int kd = 0; kd < DH / 32; ++kd) {
        if (ok) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(q_nope + qrow * DH + kd * 32 + q4 * 4);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(q_nope + qrow * DH + kd * 32 + 16 + q4 * 4);
            qb[kd] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
            qb[kd] = zero_bf16x8();
        }
    }

    // A operand lane (q4, r16), k-step kd: W_UK[d(kd, q4, e)][r0 + 16mt + r16], e = 0..7
    const u16* abase = wt + (4 * q4 + (r16 >> 2)) * PRO_STRIDE + 4 * (r16 & 3);
#pragma unroll 4
    for (int mt = 0; mt < PRO_COLS / 16; ++mt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < DH / 32; ++kd) {
            const u16* pa = abase + kd * 32 * PRO_STRIDE + mt * 16;
            const u32x2 lo = lds_read_tr16(pa);
            const u32x2 hi = lds_read_tr16(pa + 16 * PRO_STRIDE);
            acc = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), qb[kd], acc);
        }
        if (ok) {
            u32x2 o;
            o[0] = pack2h(acc[0] * scale_log2, acc[1] * scale_log2);
            o[1] = pack2h(acc[2] * scale_log2, acc[3] * scale_log2);
            *reinterpret_cast<u32x2*>(dst + r0 + mt * 16 + q4 * 4) = o;
        }
    }
    if (ok && blockIdx.z == 0) {
        // q^R: 64 elements = 8 chunks of 16 bytes; lane group q4 scales chunks q4 and q4 + 4
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int off = (q4 + 4 * c) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(q_rope + qrow * DR + off);
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = pack2h(__uint_as_float(v[k] << 16) * scale_log2,
                              __uint_as_float(v[k] & 0xffff0000u) * scale_log2);
            *reinterpret_cast<u32x4*>(dst + RK + off) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// Latent attention.
//
// Work split.  A workgroup takes one (context chunk, sequence) pair and NW*16*RG of
// the s_q*h_q query rows; its NW waves own RG row groups of 16 rows each (the
// N = 16 side of the 16x16x32 MFMA).
//   S^T[token][row] = C_tile . q^T      (A = latent rows from LDS, B = queries)
//   U^T[col][row]  += C_tile^T . P^T    (A = latent columns from LDS, B = P)
// The softmax state of a row lives in the four lanes l%16 + 16q.  RG = 2 would let
// every operand read from LDS feed two MFMAs (half the LDS traffic per flop), but u
// then takes 256 accumulator registers per lane and the wave runs alone on its SIMD,
// where it cannot hide LDS and MFMA latency: measured on the 128-row flagship shape,
// 4 waves x 2 row groups ran about 15 % slower than 8 waves x 1, so the launcher uses
// RG = 1 (two waves per SIMD).

// Data path.  A tile (32 rows x 576, one contiguous span of HBM) goes straight
// from global memory into LDS with global_load_lds_dwordx4 (lane l of a wave
// instruction lands at base + 16 l), three buffers deep, so no registers stage it.
// Buffer slot i (16 bytes) is row i / SROW, column chunk i % SROW of a row-major tile
// with a 32-byte pad per row; on gfx950 that stride (8 x odd dwords modulo the 64
// banks) lets both the 16-byte operand reads of 16 rows and the transposing reads
// of 4 rows x 32 bytes run without bank conflicts.  Pad slots, slots of rows past the
// chunk and the spare tail slots receive an in-bounds dummy chunk.  Each wave issues
// exactly NDMA loads per tile and converts its own slots from bf16 to fp16 in place
// once they have landed (fp16 keeps 10 mantissa bits for the kernel-rounded operands:
// the absorbed query and P; bf16 data within fp16's range converts exactly).  One
// barrier per tile publishes the converted tile and retires the buffer the next loads
// overwrite.  Rows past the chunk hold finite dummy data and get P = 0.
//
// Softmax.  Online, with a lazily raised reference: exponentials are taken against a
// per-row reference m (log2 domain) raised only when a tile's maximum exceeds it by more
// than kLazy, so p = 2^(s - m) <= 2^kLazy, which fp16 P and fp32 sums hold as precisely as
// values <= 1.  Accumulators are rescaled only when a row that has already accumulated
// raises its reference, which after the first tiles of a chunk is rare.  Normalisation
// and log-sum-exp use the same reference, so the result is the exact softmax's.
//
// Epilogue.  u = U / l is split into two bf16 terms (hi + lo, about 16 significant bits)
// and multiplied by W_UV[j] on the bf16 MFMA, so the partial written is o (d_h wide).
//
// Grid.  One-dimensional and XCD-aware: blocks with ids 8 apart run on one XCD, so the
// nz workgroups of a (chunk, sequence) pair that needs several (s_q*h_q > NW*16*RG)
// share one L2 and the second read of every tile is an L2 hit.
// ---------------------------------------------------------------------------
constexpr float kLazy = 10.f;

struct SoftmaxState {
    float m;   // reference (log2 domain), identical in the 4 lanes of a row; -inf before any score
    float l;   // lane-partial running sum of 2^(s - m)
};

// sc[e]: log2-domain scores of the lane's 8 tokens (masked: -inf).  Returns P as the fp16
// B operand.  need: this row has accumulated under its old reference and raised it, so
// its accumulators must be multiplied by alpha before this tile's P is added.
__device__ __forceinline__ f16x8 softmax_tile(SoftmaxState& st, const float (&sc)[8], bool& need, float& alpha) {
    float mt = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mt = wave_max16x4(mt);
    const bool raise = mt > st.m + kLazy;   // false while the row has seen nothing but -inf
    need = raise && st.m != kNegInf;        // a fresh row's accumulators are still zero
    alpha = raise ? fast_exp2(st.m - mt) : 1.f;
    st.l *= alpha;
    st.m = raise ? mt : st.m;
    const float muse = (st.m == kNegInf) ? 0.f : st.m;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(sc[e] - muse);
    st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    return as_f16x8(u32x4{pack2h(p[0], p[1]), pack2h(p[2], p[3]), pack2h(p[4], p[5]), pack2h(p[6], p[7])});
}

// A operand of U^T += C^T P^T: lane (q4, r16) needs column col0 + r16 of the tile at the
// eight tokens 4q4 + e and 16 + 4q4 + e (e = 0..3), the tokens whose scores the lane
// holds.  Lane m of a 16-lane group addresses row 4q4 + m/4 (then 16 rows further),
// columns col0 + 4(m%4)..+3; the transposing read hands lane j column col0 + j.
__device__ __forceinline__ f16x8 gather_col(const u16* lds, int stride, int q4, int r16, int col0) {
    const u16* p0 = lds + (4 * q4 + (r16 >> 2)) * stride + col0 + 4 * (r16 & 3);
    const u32x2 lo = lds_read_tr16(p0);
    const u32x2 hi = lds_read_tr16(p0 + 16 * stride);
    return as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS byte address lds_base + 16 l; lds_base must be wave-uniform.  It is
// issued from inline assembly so that the compiler, which cannot tell which LDS bytes
// such a load writes, does not wait for all of them before every later LDS access;
// callers wait with wait_vmcnt<> before reading the destination.  The compiler does not
// count these loads, so its own waits on later global loads only over-wait (loads
// retire in issue order).  The global address is a wave-uniform 64-bit base (SGPRs)
// plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
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

template <int NW, int RG, int CS>
__global__ __launch_bounds__(NW * 64) void absorb_decode_kernel(
    const u16* __restrict__ qhat, const u16* __restrict__ w_uv,
    const u16* __restrict__ cache, int64_t bstride, const int32_t* __restrict__ ctx_lens,
    int max_ctx, int h_q, int g, int s_q, int chunk, int n_split, int nz, int batch,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    constexpr int STRIDE = W + 16;    // LDS row stride in elements
    constexpr int SROW = STRIDE / 8;  // 16-byte slots per LDS row (72 data + 2 pad)
    constexpr int CPR = W / 8;        // data slots per row
    constexpr int KS = W / 32;        // 18 k-steps of the score contraction
    constexpr int KL = RK / 32;       // 16 of them over the latent part (q~ in registers)
    constexpr int NU = RK / 16;       // 32 latent column tiles of U^T
    constexpr int NT = NW * 64;
    constexpr int TSLOTS = TT * SROW;              // slots of a tile
    constexpr int NDMA = (TSLOTS + NT - 1) / NT;   // direct loads per wave per tile
    constexpr int BSLOTS = NDMA * NT;              // slots of a buffer (spare tail included)
    constexpr int BROWS = (NW / CS) * 16 * RG;     // query rows of a workgroup
    constexpr int NUW = NU / CS;                   // column tiles of U^T per wave
    static_assert(NW % CS == 0 && NU % CS == 0 && (CS == 1 || RG == 1), "column split");
    constexpr int QRS = DR + 16;                   // LDS row stride of the rotary queries
    // column tile of the U loop at which conversion slot i is read, and written back
    constexpr auto cv_read = [](int i) { return i * NUW / NDMA; };
    constexpr auto cv_write = [](int i) { return i * NUW / NDMA + 2 < NUW ? i * NUW / NDMA + 2 : NUW - 1; };
    // three separately declared buffers: with the tile loop unrolled by three every
    // access names a fixed buffer, so the compiler can tell that reading one buffer
    // does not depend on the direct loads still landing in the others
    __shared__ __attribute__((aligned(16))) u16 buf0[BSLOTS * 8];
    __shared__ __attribute__((aligned(16))) u16 buf1[BSLOTS * 8];
    __shared__ __attribute__((aligned(16))) u16 buf2[BSLOTS * 8];
    __shared__ __attribute__((aligned(16))) u16 qr_lds[BROWS * QRS];

    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int z = slot % nz;
    const int pair = (slot / nz) * 8 + xcd;
    if (pair >= n_split * batch) return;           // padding of the last group of 8
    // pair = p * batch + bb with b = (bb + p) mod batch: the sequence index varies fastest
    // across XCDs and chunk p of sequence b runs on XCD (b + p) % 8, so ragged batches
    // spread evenly (chunk-major numbering would put every sequence's first, always full,
    // chunk on the same XCD when n_split is a multiple of 8)
    const int p = pair / batch, bb = pair - p * batch;
    const int b = bb + p % batch < batch ? bb + p % batch : bb + p % batch - batch;
    const int L = clampi(ctx_lens[b], 0, max_ctx);
    const int t0 = p * chunk;
    if (t0 >= L) return;
    const int t1 = min(t0 + chunk, L);
    const int ntiles = (t1 - t0 + TT - 1) / TT;
    // tokens below t_full are visible to every query row and inside the chunk
    const int t_full = min(t1, clampi(L - s_q + 1, 0, L));

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, r16 = lane & 15;
    const int RQ = s_q * h_q;
    const int hpg = h_q / g;
    // wave = wslot * CS + part: row slot wslot, latent column part `part` of u
    const int wslot = wave / CS, part = wave - (wave / CS) * CS;
    const int rho0 = z * BROWS + wslot * (16 * RG);  // first row of the wave
    const bool active = rho0 < RQ;
    int nvis[RG];
    bool row_ok[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int rho = rho0 + 16 * rg + r16;
        row_ok[rg] = rho < RQ;
        const int s = row_ok[rg] ? rho / h_q : 0;
        nvis[rg] = clampi(L - s_q + s + 1, 0, L);
    }

    const u16* seq = cache + (size_t)b * bstride + (size_t)t0 * W;
    // byte offset within a tile of the chunk each of this lane's load slots carries
    // (-1: pad or spare slot)
    int dma_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int sl = (i * NW + wave) * 64 + lane;
        const int r = sl / SROW, c = sl - r * SROW;
        dma_off[i] = (sl < TSLOTS && c < CPR) ? (r * W + c * 8) * 2 : -1;
    }
    // Issue the direct loads of tile `it` into the buffer at LDS byte address tbuf.
    // Tiles past the chunk are clamped to its last tile (their buffer is never read), so
    // every step issues the same number of loads and waits the same way.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto dma_tile = [&](int it, uint32_t tbuf) {
        it = min(it, ntiles - 1);
        const u16* tsrc = seq + (size_t)it * TT * W;
        const int lim = min(TT, t1 - t0 - it * TT) * W * 2;   // rows past the chunk: dummy
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const uint32_t off = (dma_off[i] >= 0 && dma_off[i] < lim) ? (uint32_t)dma_off[i] : 0u;
            dma16(tsrc, off, tbuf + (uint32_t)((i * NW + wave_s) * 1024));
        }
    };

    // absorbed latent queries in registers; the 64 rotary columns of the block's rows in
    // LDS (read once per tile per row group), published by the first tile barrier
    f16x8 qv[RG][KL];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const u16* qsrc = qhat + ((size_t)b * RQ + (row_ok[rg] ? rho0 + 16 * rg + r16 : 0)) * W + q4 * 8;
#pragma unroll
        for (int kk = 0; kk < KL; ++kk) qv[rg][kk] = row_ok[rg] ? ld_f16x8(qsrc + kk * 32) : zero_f16x8();
    }
    for (int c = tid; c < BROWS * (DR / 8); c += NT) {
        const int r = c / (DR / 8), col = c - r * (DR / 8);
        const int qrow = z * BROWS + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qrow < RQ) v = *reinterpret_cast<const u32x4*>(qhat + ((size_t)b * RQ + qrow) * W + RK + col * 8);
        *reinterpret_cast<u32x4*>(qr_lds + r * QRS + col * 8) = v;
    }

    floatx4 uacc[RG][NUW];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int n = 0; n < NUW; ++n) uacc[rg][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) st[rg] = SoftmaxState{kNegInf, 0.f};

    // One tile: (barrier) start the loads of tile it+2, compute tile it, and while the
    // U MFMAs run convert this wave's slots of tile it+1 (its loads were issued one step
    // earlier).  The barrier marks tile it converted by every wave and tile it-1, whose
    // buffer the new loads reuse, consumed by every wave.  A wave whose rows all lie
    // past s_q*h_q computes on zero queries and discards the result: every wave runs
    // the same straight-line step, so the conversion can interleave with the MFMAs.
    auto step = [&](int it, const u16* lds, uint32_t dma_buf, u16* next_lds) {
        const int tb = t0 + it * TT;
        block_sync();
        dma_tile(it + 2, dma_buf);
        f16x8 pb[RG];
        {
            floatx4 acc[RG][2];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) acc[rg][0] = acc[rg][1] = floatx4{0.f, 0.f, 0.f, 0.f};
            const u16* arow = lds + r16 * STRIDE + q4 * 8;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const f16x8 a0 = ld_f16x8(arow + kk * 32);
                const f16x8 a1 = ld_f16x8(arow + 16 * STRIDE + kk * 32);
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    const f16x8 bq = kk < KL ? qv[rg][kk]
                                             : ld_f16x8(qr_lds + (wslot * 16 * RG + 16 * rg + r16) * QRS +
                                                        (kk - KL) * 32 + q4 * 8);
                    acc[rg][0] = mfma16h(a0, bq, acc[rg][0]);
                    acc[rg][1] = mfma16h(a1, bq, acc[rg][1]);
                }
                // bound how far the scheduler hoists operand reads (register pressure)
                if (kk % 6 == 5) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                float sc[8];
                if (tb + TT <= t_full) {
#pragma unroll
                    for (int th = 0; th < 2; ++th)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sc[th * 4 + i] = acc[rg][th][i];
                } else {
#pragma unroll
                    for (int th = 0; th < 2; ++th)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = tb + th * 16 + q4 * 4 + i;
                            sc[th * 4 + i] = (row_ok[rg] && t < t1 && t < nvis[rg]) ? acc[rg][th][i] : kNegInf;
                        }
                }
                bool need;
                float alpha;
                pb[rg] = softmax_tile(st[rg], sc, need, alpha);
                if (__builtin_expect(__any(need), 0)) {
                    // rare: kept as a real branch so the accumulators are not touched on
                    // the common path
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int n = 0; n < NUW; ++n) uacc[rg][n] *= alpha;
                }
            }
        }
        wait_vmcnt<NDMA>();   // this wave's loads of tile it+1 have landed
        // U MFMAs, with the conversion of this wave's NDMA slots of tile it+1 spread over
        // them: slot i is read at column tile cv_read(i) and written back converted two
        // column tiles later, so only a few slots are held in registers at a time
        u32x4 cv[NDMA];
#pragma unroll
        for (int n = 0; n < NUW; ++n) {
#pragma unroll
            for (int i = 0; i < NDMA; ++i)
                if (cv_read(i) == n)
                    cv[i] = *reinterpret_cast<const u32x4*>(next_lds + ((i * NW + wave) * 64 + lane) * 8);
            const f16x8 a = gather_col(lds, STRIDE, q4, r16, 16 * (part * NUW + n));
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) uacc[rg][n] = mfma16h(a, pb[rg], uacc[rg][n]);
#pragma unroll
            for (int i = 0; i < NDMA; ++i)
                if (cv_write(i) == n)
                    *reinterpret_cast<u32x4*>(next_lds + ((i * NW + wave) * 64 + lane) * 8) = bf8_to_h8(cv[i]);
            if (n % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
    };

    const uint32_t a0 = lds_addr(buf0), a1 = lds_addr(buf1), a2 = lds_addr(buf2);
    dma_tile(0, a0);
    dma_tile(1, a1);
    wait_vmcnt<NDMA>();
    {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            u16* ptr = buf0 + ((i * NW + wave) * 64 + lane) * 8;
            *reinterpret_cast<u32x4*>(ptr) = bf8_to_h8(*reinterpret_cast<const u32x4*>(ptr));
        }
    }
    for (int it = 0; it < ntiles; it += 3) {
        step(it, buf0, a2, buf1);
        if (it + 1 < ntiles) step(it + 1, buf1, a0, buf2);
        if (it + 2 < ntiles) step(it + 2, buf2, a1, buf0);
    }
    // no direct load may still be writing this workgroup's LDS when it ends
    wait_vmcnt<0>();
    if constexpr (CS == 1) {
        if (!active) return;

#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int rho = rho0 + 16 * rg + r16;
            const int s = row_ok[rg] ? rho / h_q : 0;
            const int h = row_ok[rg] ? rho - s * h_q : 0;
            const float l = wave_sum16x4(st[rg].l);
            const float inv = l > 0.f ? 1.f / l : 0.f;
            // U^T as the B operand of o^T = W_UV[j] U^T: k-step ks covers latent columns
            // 32ks + (token slot order of P), which are uacc[2ks + e/4][e%4] of this lane
            bf16x8 ub[RK / 32], ul[RK / 32];
#pragma unroll
            for (int ks = 0; ks < RK / 32; ++ks) {
                u32x4 vh, vl;
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const floatx4& src = uacc[rg][2 * ks + (hh >> 1)];
                    const float a = src[2 * (hh & 1)] * inv, c = src[2 * (hh & 1) + 1] * inv;
                    const u16 ah = f2bf(a), ch = f2bf(c);
                    vh[hh] = pack2(ah, ch);
                    vl[hh] = pack2f(a - bf2f(ah), c - bf2f(ch));
                }
                ub[ks] = as_bf16x8(vh);
                ul[ks] = as_bf16x8(vl);
            }
            const int jrow = h / hpg;
            const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
            // groups of the row group's 16 rows (they never straddle a query token: h_q % 16 == 0)
            const int first = rho0 + 16 * rg;
            const int last = min(first + 15, RQ - 1);
            if (first > last) continue;
            const int jlo = (first % h_q) / hpg, jhi = (last % h_q) / hpg;
            for (int jj = jlo; jj <= jhi; ++jj) {
                const u16* wj = w_uv + (size_t)jj * DH * RK;
#pragma unroll 2
                for (int mt = 0; mt < DH / 16; ++mt) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                    const u16* wrow = wj + (size_t)(mt * 16 + r16) * RK + q4 * 4;
#pragma unroll
                    for (int ks = 0; ks < RK / 32; ++ks) {
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(wrow + ks * 32);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(wrow + ks * 32 + 16);
                        const bf16x8 wa = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                        acc = mfma16(wa, ub[ks], acc);
                        acc = mfma16(wa, ul[ks], acc);
                    }
                    if (row_ok[rg] && jrow == jj) *reinterpret_cast<floatx4*>(part_o + prow * DH + mt * 16 + q4 * 4) = acc;
                }
            }
            if (row_ok[rg] && q4 == 0) part_lse[prow] = l > 0.f ? (st[rg].m + __log2f(l)) * kLn2 : kNegInf;
        }
    } else {
        // Column-split epilogue (one row group per wave).  The wave holds u for its 16 rows
        // over latent columns [part * RK / CS, (part + 1) * RK / CS), so its W_UV product
        // is a partial sum over those columns; the CS partials of a row slot meet in LDS
        // (the tile buffers, free once every wave has passed the barrier below) and each
        // wave of the slot sums and writes every CS-th 16-wide block of d_h.
        block_sync();
        constexpr int KSW = NUW / 2;   // k-steps of the wave's columns
        const int rho = rho0 + r16;
        const bool rok = row_ok[0];
        const int s = rok ? rho / h_q : 0;
        const int h = rok ? rho - s * h_q : 0;
        const float l = wave_sum16x4(st[0].l);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        bf16x8 ub[KSW], ul[KSW];
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            u32x4 vh, vl;
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const floatx4& src = uacc[0][2 * ks + (hh >> 1)];
                const float x = src[2 * (hh & 1)] * inv, y = src[2 * (hh & 1) + 1] * inv;
                const u16 xh = f2bf(x), yh = f2bf(y);
                vh[hh] = pack2(xh, yh);
                vl[hh] = pack2f(x - bf2f(xh), y - bf2f(yh));
            }
            ub[ks] = as_bf16x8(vh);
            ul[ks] = as_bf16x8(vl);
        }
        const int jrow = h / hpg;
        floatx4 ores[DH / 16];
#pragma unroll
        for (int mt = 0; mt < DH / 16; ++mt) ores[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (active) {
            const int first = rho0;
            const int last = min(first + 15, RQ - 1);
            const int jlo = (first % h_q) / hpg, jhi = (last % h_q) / hpg;
            for (int jj = jlo; jj <= jhi; ++jj) {
                const u16* wj = w_uv + (size_t)jj * DH * RK + part * (RK / CS);
#pragma unroll
                for (int mt = 0; mt < DH / 16; ++mt) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                    const u16* wrow = wj + (size_t)(mt * 16 + r16) * RK + q4 * 4;
#pragma unroll
                    for (int ks = 0; ks < KSW; ++ks) {
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(wrow + ks * 32);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(wrow + ks * 32 + 16);
                        const bf16x8 wa = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                        acc = mfma16(wa, ub[ks], acc);
                        acc = mfma16(wa, ul[ks], acc);
                    }
                    if (jrow == jj) ores[mt] = acc;
                }
            }
        }
        // partial of wave w, block mt: buffer mt / 4, floatx4 slot (w * 4 + mt % 4) * 64 + lane
        float* red0 = reinterpret_cast<float*>(buf0);
        float* red1 = reinterpret_cast<float*>(buf1);
        static_assert(NW * 4 * 64 * 16 <= (int)sizeof(buf0), "partials fit in a tile buffer");
#pragma unroll
        for (int mt = 0; mt < DH / 16; ++mt)
            *reinterpret_cast<floatx4*>((mt < 4 ? red0 : red1) + ((wave * 4 + (mt & 3)) * 64 + lane) * 4) = ores[mt];
        block_sync();
        if (active && rok) {
            const size_t prow = ((size_t)p * batch * s_q + (size_t)b * s_q + s) * h_q + h;
            for (int mt = part; mt < DH / 16; mt += CS) {
                floatx4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < CS; ++c)
                    sum += *reinterpret_cast<const floatx4*>((mt < 4 ? red0 : red1) +
                                                             (((wslot * CS + c) * 4 + (mt & 3)) * 64 + lane) * 4);
                *reinterpret_cast<floatx4*>(part_o + prow * DH + mt * 16 + q4 * 4) = sum;
            }
            if (part == 0 && q4 == 0) part_lse[prow] = l > 0.f ? (st[0].m + __log2f(l)) * kLn2 : kNegInf;
        }
    }
}

template <int NW, int RG, int CS>
hipError_t launch_absorb_t(const DecodeArgs& a, int nz, hipStream_t st) {
    const int pairs = a.n_split * a.batch;
    dim3 grid(((pairs + 7) / 8) * 8 * nz);
    hipLaunchKernelGGL((absorb_decode_kernel<NW, RG, CS>), grid, dim3(NW * 64), 0, st, (const u16*)a.qhat,
                       (const u16*)a.w_uv, (const u16*)a.cache, a.bstride, a.ctx_lens, a.max_ctx, a.h_q, a.g,
                       a.s_q, a.chunk, a.n_split, nz, a.batch, a.part_o, a.part_lse);
    return hipGetLastError();
}

}  // namespace

int absorb_block_rows(int query_rows) { return query_rows <= 32 ? 32 : (query_rows <= 64 ? 64 : 128); }

hipError_t launch_absorb_bf16(const DecodeArgs& a, hipStream_t st) {
    const int hpg = a.h_q / a.g;
    const int rows_per_group = a.batch * a.s_q * hpg;
    dim3 pgrid((rows_per_group + 63) / 64, a.g, RK / PRO_COLS);
    hipLaunchKernelGGL(absorb_prologue_kernel, pgrid, dim3(256), 0, st,
                       (const u16*)a.q_nope, (const u16*)a.q_rope, (const u16*)a.w_uk, (u16*)a.qhat,
                       a.batch, a.h_q, a.g, a.s_q, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int RQ = a.s_q * a.h_q;
    const int rows = absorb_block_rows(RQ);
    const int nz = (RQ + rows - 1) / rows;
    e = record_if(a.ev_before, st);
    if (e != hipSuccess) return e;
    if (rows == 32) {
        e = launch_absorb_t<8, 1, 4>(a, nz, st);
    } else if (rows == 64) {
        e = launch_absorb_t<8, 1, 2>(a, nz, st);
    } else {
        e = launch_absorb_t<8, 1, 1>(a, nz, st);
    }
    if (e != hipSuccess) return e;
    return record_if(a.ev_after, st);
}

}  // namespace gqla
