// C-ABI host layer of libgqla: argument validation, split-K planning, workspace
// layout and kernel launches on the caller's stream.  Declarations and the
// contract of each entry point are in include/gqla.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/gqla.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

gqla_status fail(gqla_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

gqla_status ok() {
    g_err[0] = '\0';
    return GQLA_OK;
}

// Compute units of the current device, cached per device id.  Concurrent first calls
// may both query the attribute; they store the same value, and the atomics make the
// cache safe to read and write from several threads.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Device-resident scratch of gqla_decode_gqa_noalloc: the split-K partials of a call
// live here instead of in a caller workspace.  Every device the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken once per device with
// hipGetSymbolAddress (on that device's first no-allocation call, with the device
// current) and only that address is ever handed to kernels.
constexpr size_t kNoAllocScratchBytes = GQLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[64];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_bf16_mfma_shape(const gqla_shape& s) { return s.r_kv == 512 && s.d_r == 64 && s.d_h == 128; }

gqla_status check_shape(const gqla_shape* sp, int path) {
    if (!sp) return fail(GQLA_ERR_INVALID_ARG, "shape is null");
    const gqla_shape& s = *sp;
    if (path != GQLA_PATH_ABSORB && path != GQLA_PATH_GQA && path != GQLA_PATH_SPARSE)
        return fail(GQLA_ERR_INVALID_ARG, "path %d is none of absorb (0), gqa (1), sparse (2)", path);
    if (s.h_q <= 0 || s.g <= 0 || s.r_kv <= 0 || s.d_r <= 0 || s.d_h <= 0)
        return fail(GQLA_ERR_INVALID_ARG, "dims must be positive (h_q=%d g=%d r_kv=%d d_r=%d d_h=%d)", s.h_q, s.g, s.r_kv, s.d_r, s.d_h);
    if (s.h_q % s.g != 0) return fail(GQLA_ERR_INVALID_ARG, "h_q=%d is not a multiple of g=%d", s.h_q, s.g);
    if (s.s_q < 1 || s.s_q > 4) return fail(GQLA_ERR_INVALID_ARG, "s_q=%d outside 1..4", s.s_q);
    if (!(s.scale > 0.f) || !std::isfinite(s.scale)) return fail(GQLA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (s.r_kv % 8 || s.d_r % 8 || s.d_h % 8) return fail(GQLA_ERR_INVALID_ARG, "r_kv, d_r and d_h must be multiples of 8");
    if (s.dtype == GQLA_BF16) {
        if (!is_bf16_mfma_shape(s))
            return fail(GQLA_ERR_UNSUPPORTED, "bf16 kernels are built for r_kv=512, d_r=64, d_h=128 (got %d, %d, %d)", s.r_kv, s.d_r, s.d_h);
        if (path == GQLA_PATH_ABSORB && s.h_q % 16 != 0)
            return fail(GQLA_ERR_UNSUPPORTED, "bf16 absorb path needs h_q %% 16 == 0 (got %d)", s.h_q);
        if (path == GQLA_PATH_GQA && !gqla::gqa_bf16_supported(s.g, s.s_q * (s.h_q / s.g)))
            return fail(GQLA_ERR_UNSUPPORTED, "bf16 GQA path is built for g in {1,2,4,8} (got %d)", s.g);
    } else if (s.dtype == GQLA_F32) {
        if (s.r_kv > 1024 || s.d_r > 256 || s.d_h > 256)
            return fail(GQLA_ERR_UNSUPPORTED, "fp32 kernels need r_kv <= 1024, d_r <= 256, d_h <= 256");
    } else {
        return fail(GQLA_ERR_INVALID_ARG, "unknown dtype %d", s.dtype);
    }
    return GQLA_OK;
}

struct Plan {
    int n_split, chunk;
};

// Context chunking.  Chunks are multiples of the bf16 token tile; the fp32 path keeps
// a chunk's scores in LDS, so its chunks are capped.  Automatic mode aims for at
// least one workgroup per compute unit and chunks of at most 4096 tokens (so ragged
// batches spread over the CUs); an explicit num_splits is an upper bound on chunks.
Plan plan(const gqla_shape& s, int path, int batch, int max_ctx, int num_splits) {
    const int align = s.dtype == GQLA_BF16 ? gqla::kBf16TokenTile : 1;
    const int ctx = max_ctx > 0 ? max_ctx : 1;
    int want;
    if (num_splits > 0) {
        want = num_splits;
    } else {
        int units = batch > 0 ? batch : 1;
        int per_cu = 1;                                 // work units wanted per compute unit
        if (s.dtype == GQLA_BF16 && path == GQLA_PATH_ABSORB) {
            const int rows = gqla::absorb_block_rows(s.s_q * s.h_q);
            units *= (s.s_q * s.h_q + rows - 1) / rows;
        } else if (s.dtype == GQLA_BF16 && path == GQLA_PATH_GQA) {
            // one 32-row tile in flight per workgroup: narrow rows (small g) need several
            // workgroups per CU to keep enough bytes in flight (measured at 8192 tokens:
            // g = 2 0.56 -> 0.67 and g = 1 0.40 -> 0.50 of peak with 4 per CU; 7 per CU
            // was slower again at g = 1)
            const size_t tile = (size_t)gqla::kBf16TokenTile * (2 * s.g * s.d_h + s.d_r) * 2;
            if (tile < (64u << 10)) per_cu = std::min(4, (int)(((140u << 10) + tile - 1) / tile));
        } else if (s.dtype == GQLA_BF16 && path == GQLA_PATH_SPARSE) {
            // one wave per (sequence, query token, group, 16-head tile): aim at 8 waves per CU
            units *= s.s_q * s.g * ((s.h_q / s.g + 15) / 16);
            per_cu = 8;
        }
        const int cus = device_cus();
        want = (cus * per_cu + units - 1) / units;
        // chunks of at most 4096 tokens (8192 on the bf16 absorb path, whose workgroups
        // hold 64 query rows and one of them fills a CU's LDS; one chunk per sequence
        // also lets its kernel write the result without a combine)
        const int max_chunk = (s.dtype == GQLA_BF16 && path == GQLA_PATH_ABSORB) ? 8192 : 4096;
        const int by_len = (ctx + max_chunk - 1) / max_chunk;
        if (by_len > want) want = by_len;
    }
    if (want > ctx) want = ctx;
    if (want < 1) want = 1;
    int chunk = (ctx + want - 1) / want;
    chunk = (chunk + align - 1) / align * align;
    if (s.dtype == GQLA_F32 && chunk > gqla::kF32MaxChunk) chunk = gqla::kF32MaxChunk;
    Plan p;
    p.chunk = chunk;
    p.n_split = (ctx + chunk - 1) / chunk;
    return p;
}

// Length-aware choice of num_splits (bf16 absorb and GQA paths).  A decode launch is
// a grid of workgroups, one per (context chunk, sequence) pair and, on the absorb
// path, per 128-row group of query rows.  Workgroups of pairs past a sequence's end
// return at once.  The candidates are the automatic plan, the "fill" plans whose grid
// is exactly k times the concurrent workgroups of the device, and the balanced plans
// with the smallest chunk whose non-empty workgroups fit k rounds (k = 1..4); the
// estimate of a plan is
//   rounds x (longest work item + overhead),
// rounds = ceil(non-empty workgroups / concurrent workgroups), with the per-workgroup
// overhead (query staging, the W_UV epilogue or output write, the partial it adds to
// the combine) in tokens: about 1000, fitted on MI355X to the absorb kernel on the
// ragged 64K-128K workload and kept for the GQA kernel, whose time there also falls
// with fewer, longer chunks (16 chunks 1082 us, 64 chunks 1166 us).  A plan with more
// chunks replaces the current choice only when it is estimated 10 % faster: the
// estimate leaves out costs that grow with the chunk count (dispatch imbalance inside
// a round, the combine's reads), and a smaller grid also needs less workspace.  Partly
// filled rounds are estimated as full because the dispatcher places workgroups
// statically (workgroup i runs on XCD i mod 8, and within an XCD by a fixed rotation),
// so one crowded group of CUs sets the time: measured at 16 sequences of 64K-128K
// tokens, 18-22 chunks per sequence (288-352 workgroups for 256 CUs, a quarter of them
// empty) ran 30-60 % slower than 16 chunks (256 workgroups).
// Work items of a plan with chunk c: sequence b gives ceil(L_b / c) items of
// roundup32(ceil(L_b / n)) tokens (the kernels' equal per-sequence chunks).
long long split_items(const int32_t* lens, int batch, int max_ctx, int chunk, int mult, int* longest_item) {
    long long units = 0;
    int longest = 0;
    for (int b = 0; b < batch; ++b) {
        const int L = std::min(std::max(lens[b], 0), max_ctx);
        const int n = (L + chunk - 1) / chunk;
        units += (long long)mult * n;
        if (n > 0) {
            const int a = gqla::kBf16TokenTile;
            longest = std::max(longest, ((L + n - 1) / n + a - 1) / a * a);
        }
    }
    if (longest_item) *longest_item = longest;
    return units;
}

double split_estimate(const int32_t* lens, int batch, int max_ctx, int chunk, int mult, int slots, double ovh) {
    int longest = 0;
    const long long units = split_items(lens, batch, max_ctx, chunk, mult, &longest);
    const long long rounds = (units + slots - 1) / slots;
    return (double)rounds * (longest + ovh);
}

struct Layout {
    size_t part_o, part_lse, qhat, wpack, total;
};

Layout layout(const gqla_shape& s, int path, int batch, const Plan& p) {
    const size_t rows = (size_t)batch * s.s_q * s.h_q;
    Layout l;
    l.part_o = 0;
    l.part_lse = align256(l.part_o + (size_t)p.n_split * rows * s.d_h * sizeof(float));
    l.qhat = align256(l.part_lse + (size_t)p.n_split * rows * sizeof(float));
    size_t end = l.qhat;
    l.wpack = l.qhat;
    if (path == GQLA_PATH_ABSORB && s.dtype == GQLA_BF16) {
        l.wpack = align256(l.qhat + rows * gqla::absorb_qrec_bytes());
        end = align256(l.wpack + gqla::absorb_wpack_bytes(s.g));
    }
    l.total = end;
    return l;
}

gqla_status check_sizes(int batch, int max_ctx) {
    if (batch < 0) return fail(GQLA_ERR_INVALID_ARG, "batch=%d < 0", batch);
    if (max_ctx < 0) return fail(GQLA_ERR_INVALID_ARG, "max_ctx=%d < 0", max_ctx);
    return GQLA_OK;
}

gqla_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(GQLA_ERR_INVALID_ARG, "%s is null", name);
    if (!aligned16(p)) return fail(GQLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return GQLA_OK;
}

gqla_status check_stride(int64_t stride, int64_t row_width, int max_ctx, const char* name) {
    if (stride % 8 != 0) return fail(GQLA_ERR_INVALID_ARG, "%s=%lld is not a multiple of 8 elements", name, (long long)stride);
    if (stride < row_width * (int64_t)max_ctx)
        return fail(GQLA_ERR_INVALID_ARG, "%s=%lld < max_ctx * row width = %lld", name, (long long)stride,
                    (long long)(row_width * (int64_t)max_ctx));
    return GQLA_OK;
}

#define TRY(x)                               \
    do {                                     \
        gqla_status _st = (x);               \
        if (_st != GQLA_OK) return _st;      \
    } while (0)

gqla_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GQLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Device address of the current device's copy of `scratch` (looked up once per device).
gqla_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(GQLA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..63", dev);
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        void* p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        slot.ptr = slot.err == hipSuccess ? p : nullptr;
    });
    if (slot.err != hipSuccess) return hip_status(slot.err, "hipGetSymbolAddress(scratch)");
    if (!slot.ptr) return fail(GQLA_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    *out = slot.ptr;
    return GQLA_OK;
}

// use_scratch: the partials go to the static device scratch instead of `workspace`
// (which is then ignored); a call needing more than its size fails before any launch.
gqla_status decode_common(int path, const gqla_shape* sp, int32_t batch, int32_t max_ctx, const void* q_nope,
                          const void* q_rope, const void* w_uk, const void* w_uv, const void* cache,
                          int64_t bstride, const int32_t* ctx_lens, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, int32_t num_splits, void* stream, bool use_scratch = false) {
    TRY(check_shape(sp, path));
    TRY(check_sizes(batch, max_ctx));
    if (num_splits < 0) return fail(GQLA_ERR_INVALID_ARG, "num_splits=%d < 0", num_splits);
    const gqla_shape& s = *sp;
    if (batch == 0) return ok();
    const int64_t width = path == GQLA_PATH_ABSORB ? s.r_kv + s.d_r : 2LL * s.g * s.d_h + s.d_r;
    TRY(check_ptr(q_nope, "q_nope"));
    TRY(check_ptr(q_rope, "q_rope"));
    if (path == GQLA_PATH_ABSORB) {
        TRY(check_ptr(w_uk, "w_uk"));
        TRY(check_ptr(w_uv, "w_uv"));
    }
    TRY(check_ptr(cache, path == GQLA_PATH_ABSORB ? "latent" : "group_cache"));
    TRY(check_stride(bstride, width, max_ctx, path == GQLA_PATH_ABSORB ? "latent_bstride" : "group_bstride"));
    if (!ctx_lens) return fail(GQLA_ERR_INVALID_ARG, "ctx_lens is null");
    TRY(check_ptr(out, "out"));
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(GQLA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
    const Plan p = plan(s, path, batch, max_ctx, num_splits);
    const Layout lay = layout(s, path, batch, p);
    if (use_scratch) {
        if (lay.total > kNoAllocScratchBytes)
            return fail(GQLA_ERR_WORKSPACE,
                        "the call needs %zu bytes of scratch, above the static maximum of %zu "
                        "(use fewer sequences per call or a smaller num_splits)",
                        lay.total, kNoAllocScratchBytes);
        TRY(scratch_address(&workspace));
    } else {
        if (!workspace) return fail(GQLA_ERR_WORKSPACE, "workspace is null (%zu bytes needed)", lay.total);
        if (!aligned16(workspace)) return fail(GQLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
        if (workspace_bytes < lay.total)
            return fail(GQLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, lay.total);
    }

    gqla::DecodeArgs a;
    a.h_q = s.h_q;
    a.g = s.g;
    a.r_kv = s.r_kv;
    a.d_r = s.d_r;
    a.d_h = s.d_h;
    a.s_q = s.s_q;
    a.scale = s.scale;
    a.batch = batch;
    a.max_ctx = max_ctx;
    a.n_split = p.n_split;
    a.chunk = p.chunk;
    a.cus = device_cus();
    a.q_nope = q_nope;
    a.q_rope = q_rope;
    a.w_uk = w_uk;
    a.w_uv = w_uv;
    a.cache = cache;
    a.bstride = bstride;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws + lay.part_o);
    a.part_lse = reinterpret_cast<float*>(ws + lay.part_lse);
    a.qhat = ws + lay.qhat;
    a.wpack = ws + lay.wpack;
    a.ev_before = g_ev_before;
    a.ev_after = g_ev_after;

    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (s.dtype == GQLA_BF16) {
        e = path == GQLA_PATH_ABSORB ? gqla::launch_absorb_bf16(a, st) : gqla::launch_gqa_bf16(a, st);
    } else {
        e = path == GQLA_PATH_ABSORB ? gqla::launch_absorb_f32(a, st) : gqla::launch_gqa_f32(a, st);
    }
    if (e != hipSuccess) return hip_status(e, "decode launch");
    // the bf16 absorb kernel writes the result itself when each sequence is one chunk
    if (s.dtype == GQLA_BF16 && path == GQLA_PATH_ABSORB && p.n_split == 1) return ok();
    return hip_status(gqla::launch_combine(a, s.dtype == GQLA_BF16, st), "combine launch");
}

}  // namespace

extern "C" {

gqla_status gqla_workspace_size(const gqla_shape* shape, int32_t path, int32_t batch, int32_t max_ctx,
                                int32_t num_splits, size_t* bytes) {
    TRY(check_shape(shape, path));
    TRY(check_sizes(batch, max_ctx));
    if (num_splits < 0) return fail(GQLA_ERR_INVALID_ARG, "num_splits=%d < 0", num_splits);
    if (!bytes) return fail(GQLA_ERR_INVALID_ARG, "bytes is null");
    const Plan p = plan(*shape, path, batch, max_ctx, num_splits);
    *bytes = layout(*shape, path, batch, p).total;
    return ok();
}

gqla_status gqla_plan_splits(const gqla_shape* shape, int32_t path, int32_t batch, int32_t max_ctx,
                             int32_t num_splits, int32_t* n_split, int32_t* chunk) {
    TRY(check_shape(shape, path));
    TRY(check_sizes(batch, max_ctx));
    if (num_splits < 0) return fail(GQLA_ERR_INVALID_ARG, "num_splits=%d < 0", num_splits);
    if (!n_split || !chunk) return fail(GQLA_ERR_INVALID_ARG, "n_split or chunk is null");
    const Plan p = plan(*shape, path, batch, max_ctx, num_splits);
    *n_split = p.n_split;
    *chunk = p.chunk;
    return ok();
}

gqla_status gqla_plan_splits_lens(const gqla_shape* shape, int32_t path, int32_t batch, int32_t max_ctx,
                                  const int32_t* host_ctx_lens, int32_t* num_splits, int32_t* n_split,
                                  int32_t* chunk) {
    TRY(check_shape(shape, path));
    TRY(check_sizes(batch, max_ctx));
    if (!host_ctx_lens && batch > 0) return fail(GQLA_ERR_INVALID_ARG, "host_ctx_lens is null");
    if (!num_splits || !n_split || !chunk) return fail(GQLA_ERR_INVALID_ARG, "num_splits, n_split or chunk is null");
    const gqla_shape& s = *shape;
    int best = 0;
    if (s.dtype == GQLA_BF16 && (path == GQLA_PATH_ABSORB || path == GQLA_PATH_GQA) && batch > 0 && max_ctx > 0) {
        int mult = 1, per_cu = 1;
        // per-workgroup overhead in tokens: the absorb workgroup also stages its queries,
        // fills a two-tile pipeline and runs the W_UV epilogue for 64 rows
        const double ovh = path == GQLA_PATH_ABSORB ? 4000.0 : 1000.0;
        if (path == GQLA_PATH_ABSORB) {
            const int rows = gqla::absorb_block_rows(s.s_q * s.h_q);
            mult = (s.s_q * s.h_q + rows - 1) / rows;
        } else {
            const size_t tile = (size_t)gqla::kBf16TokenTile * (2 * s.g * s.d_h + s.d_r) * 2;
            if (tile < (64u << 10)) per_cu = std::min(4, (int)(((140u << 10) + tile - 1) / tile));
        }
        const int slots = device_cus() * per_cu;
        const int auto_chunk = plan(s, path, batch, max_ctx, 0).chunk;
        long long auto_units = 0;
        for (int b = 0; b < batch; ++b)
            auto_units +=
                (long long)mult * ((std::min(std::max(host_ctx_lens[b], 0), max_ctx) + auto_chunk - 1) / auto_chunk);
        // with four or more rounds of workgroups, partial rounds and short last chunks are
        // a small share of the time and the automatic plan stands
        if (auto_units < 4LL * slots) {
            // candidates (num_splits argument, chunks per sequence), fewest chunks first
            int cand_w[9], cand_n[9], nc = 0;
            const long long fill = slots / ((long long)batch * mult);   // chunks per sequence, one round
            for (int k = 1; fill > 0 && k <= 4; ++k) {
                const int w = (int)(k * fill);
                const Plan pl = plan(s, path, batch, max_ctx, w);
                // chunk alignment can round the count up past the grid of k rounds
                if ((long long)pl.n_split * batch * mult > (long long)k * slots) continue;
                cand_w[nc] = w;
                cand_n[nc++] = pl.n_split;
            }
            // balanced plans: the smallest chunk whose work items (empty chunks of short
            // sequences are no items) fit k rounds; items of one sequence are of equal
            // size, so with ragged lengths these fill the rounds more evenly than a grid
            // of k rounds of chunks
            const int w_max = std::max(1, (max_ctx + gqla::kBf16TokenTile - 1) / gqla::kBf16TokenTile);
            for (int k = 1; k <= 4; ++k) {
                auto fits = [&](int w) {
                    return split_items(host_ctx_lens, batch, max_ctx, plan(s, path, batch, max_ctx, w).chunk, mult,
                                       nullptr) <= (long long)k * slots;
                };
                if (!fits(1)) continue;
                int lo = 1, hi = w_max;   // fits(lo); largest w that fits
                while (lo < hi) {
                    const int mid = lo + (hi - lo + 1) / 2;
                    if (fits(mid)) lo = mid;
                    else hi = mid - 1;
                }
                cand_w[nc] = lo;
                cand_n[nc++] = plan(s, path, batch, max_ctx, lo).n_split;
            }
            cand_w[nc] = 0;
            cand_n[nc++] = plan(s, path, batch, max_ctx, 0).n_split;
            for (int i = 1; i < nc; ++i)
                for (int j = i; j > 0 && cand_n[j] < cand_n[j - 1]; --j) {
                    std::swap(cand_n[j], cand_n[j - 1]);
                    std::swap(cand_w[j], cand_w[j - 1]);
                }
            double best_est = 0.0;
            for (int i = 0; i < nc; ++i) {
                const double est =
                    split_estimate(host_ctx_lens, batch, max_ctx, plan(s, path, batch, max_ctx, cand_w[i]).chunk, mult,
                                   slots, ovh);
                if (i == 0 || est < best_est * 0.9) {
                    best = cand_w[i];
                    best_est = est;
                }
            }
        }
    }
    const Plan p = plan(s, path, batch, max_ctx, best);
    *num_splits = best;
    *n_split = p.n_split;
    *chunk = p.chunk;
    return ok();
}

gqla_status gqla_expand_groups(const gqla_shape* shape, int32_t batch, int32_t max_ctx, const void* latent,
                               int64_t latent_bstride, const void* w_uk, const void* w_uv, const int32_t* ctx_lens,
                               int32_t row_begin, void* group_cache, int64_t group_bstride, void* stream) {
    TRY(check_shape(shape, GQLA_PATH_GQA));
    TRY(check_sizes(batch, max_ctx));
    const gqla_shape& s = *shape;
    if (row_begin < 0) return fail(GQLA_ERR_INVALID_ARG, "row_begin=%d < 0", row_begin);
    if (batch == 0 || row_begin >= max_ctx) return ok();
    TRY(check_ptr(latent, "latent"));
    TRY(check_ptr(w_uk, "w_uk"));
    TRY(check_ptr(w_uv, "w_uv"));
    TRY(check_ptr(group_cache, "group_cache"));
    if (!ctx_lens) return fail(GQLA_ERR_INVALID_ARG, "ctx_lens is null");
    TRY(check_stride(latent_bstride, s.r_kv + s.d_r, max_ctx, "latent_bstride"));
    TRY(check_stride(group_bstride, 2LL * s.g * s.d_h + s.d_r, max_ctx, "group_bstride"));
    gqla::ExpandArgs a;
    a.h_q = s.h_q;
    a.g = s.g;
    a.r_kv = s.r_kv;
    a.d_r = s.d_r;
    a.d_h = s.d_h;
    a.batch = batch;
    a.max_ctx = max_ctx;
    a.row_begin = row_begin;
    a.latent = latent;
    a.latent_bstride = latent_bstride;
    a.w_uk = w_uk;
    a.w_uv = w_uv;
    a.ctx_lens = ctx_lens;
    a.group_cache = group_cache;
    a.group_bstride = group_bstride;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = s.dtype == GQLA_BF16 ? gqla::launch_expand_bf16(a, st) : gqla::launch_expand_f32(a, st);
    return hip_status(e, "expand launch");
}

gqla_status gqla_decode_absorb(const gqla_shape* shape, int32_t batch, int32_t max_ctx, const void* q_nope,
                               const void* q_rope, const void* w_uk, const void* w_uv, const void* latent,
                               int64_t latent_bstride, const int32_t* ctx_lens, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream) {
    return decode_common(GQLA_PATH_ABSORB, shape, batch, max_ctx, q_nope, q_rope, w_uk, w_uv, latent,
                         latent_bstride, ctx_lens, out, lse, workspace, workspace_bytes, num_splits, stream);
}

gqla_status gqla_decode_gqa(const gqla_shape* shape, int32_t batch, int32_t max_ctx, const void* q_nope,
                            const void* q_rope, const void* group_cache, int64_t group_bstride,
                            const int32_t* ctx_lens, void* out, float* lse, void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream) {
    return decode_common(GQLA_PATH_GQA, shape, batch, max_ctx, q_nope, q_rope, nullptr, nullptr, group_cache,
                         group_bstride, ctx_lens, out, lse, workspace, workspace_bytes, num_splits, stream);
}

gqla_status gqla_decode_gqa_noalloc(const gqla_shape* shape, int32_t batch, int32_t max_ctx, const void* q_nope,
                                    const void* q_rope, const void* group_cache, int64_t group_bstride,
                                    const int32_t* ctx_lens, void* out, float* lse, int32_t num_splits,
                                    void* stream) {
    return decode_common(GQLA_PATH_GQA, shape, batch, max_ctx, q_nope, q_rope, nullptr, nullptr, group_cache,
                         group_bstride, ctx_lens, out, lse, nullptr, 0, num_splits, stream, true);
}

gqla_status gqla_decode_gqa_sparse(const gqla_shape* shape, int32_t batch, int32_t max_ctx, const void* q_nope,
                                   const void* q_rope, const void* group_cache, int64_t group_bstride,
                                   const int32_t* ctx_lens, const int32_t* indices, int32_t topk, void* out,
                                   float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                   void* stream) {
    TRY(check_shape(shape, GQLA_PATH_SPARSE));
    TRY(check_sizes(batch, max_ctx));
    if (topk < 0) return fail(GQLA_ERR_INVALID_ARG, "topk=%d < 0", topk);
    if (num_splits < 0) return fail(GQLA_ERR_INVALID_ARG, "num_splits=%d < 0", num_splits);
    const gqla_shape& s = *shape;
    if (batch == 0) return ok();
    TRY(check_ptr(q_nope, "q_nope"));
    TRY(check_ptr(q_rope, "q_rope"));
    TRY(check_ptr(group_cache, "group_cache"));
    TRY(check_stride(group_bstride, 2LL * s.g * s.d_h + s.d_r, max_ctx, "group_bstride"));
    if (!ctx_lens) return fail(GQLA_ERR_INVALID_ARG, "ctx_lens is null");
    if (topk > 0 && !indices) return fail(GQLA_ERR_INVALID_ARG, "indices is null");
    if (indices && (reinterpret_cast<uintptr_t>(indices) & 3u)) return fail(GQLA_ERR_INVALID_ARG, "indices is not 4-byte aligned");
    TRY(check_ptr(out, "out"));
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(GQLA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
    const Plan p = plan(s, GQLA_PATH_SPARSE, batch, topk, num_splits);
    const Layout lay = layout(s, GQLA_PATH_SPARSE, batch, p);
    if (!workspace) return fail(GQLA_ERR_WORKSPACE, "workspace is null (%zu bytes needed)", lay.total);
    if (!aligned16(workspace)) return fail(GQLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < lay.total)
        return fail(GQLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, lay.total);
    gqla::DecodeArgs a;
    a.h_q = s.h_q;
    a.g = s.g;
    a.r_kv = s.r_kv;
    a.d_r = s.d_r;
    a.d_h = s.d_h;
    a.s_q = s.s_q;
    a.scale = s.scale;
    a.batch = batch;
    a.max_ctx = max_ctx;
    a.n_split = p.n_split;
    a.chunk = p.chunk;
    a.q_nope = q_nope;
    a.q_rope = q_rope;
    a.w_uk = nullptr;
    a.w_uv = nullptr;
    a.cache = group_cache;
    a.bstride = group_bstride;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws + lay.part_o);
    a.part_lse = reinterpret_cast<float*>(ws + lay.part_lse);
    a.qhat = nullptr;
    a.wpack = nullptr;
    a.ev_before = g_ev_before;
    a.ev_after = g_ev_after;
    a.n_merge = p.n_split;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool bf16 = s.dtype == GQLA_BF16;
    TRY(hip_status(gqla::launch_gqa_sparse(a, indices, topk, bf16, st), "sparse decode launch"));
    return hip_status(gqla::launch_combine(a, bf16, st), "combine launch");
}

gqla_status gqla_append_rows(const gqla_shape* shape, int32_t batch, int32_t max_ctx, const void* c_new,
                             const void* kr_new, const void* q_rope_raw, void* q_rope_out, float rope_theta,
                             const int32_t* ctx_lens, void* latent, int64_t latent_bstride, const void* w_uk,
                             const void* w_uv, void* group_cache, int64_t group_bstride, void* stream) {
    // the group layout checks of the GQA path apply when new rows are expanded
    TRY(check_shape(shape, group_cache ? GQLA_PATH_GQA : GQLA_PATH_ABSORB));
    TRY(check_sizes(batch, max_ctx));
    const gqla_shape& s = *shape;
    if (s.d_r % 2) return fail(GQLA_ERR_INVALID_ARG, "d_r=%d is odd", s.d_r);
    if (s.d_r > 256) return fail(GQLA_ERR_UNSUPPORTED, "d_r=%d > 256", s.d_r);
    if (!(rope_theta > 0.f) || !std::isfinite(rope_theta))
        return fail(GQLA_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
    if ((q_rope_raw == nullptr) != (q_rope_out == nullptr))
        return fail(GQLA_ERR_INVALID_ARG, "q_rope_raw and q_rope_out must both be set or both be null");
    if (batch == 0 || max_ctx == 0) return ok();
    TRY(check_ptr(c_new, "c_new"));
    TRY(check_ptr(kr_new, "kr_new"));
    if (q_rope_raw) {
        TRY(check_ptr(q_rope_raw, "q_rope_raw"));
        TRY(check_ptr(q_rope_out, "q_rope_out"));
        if (q_rope_raw == q_rope_out) return fail(GQLA_ERR_INVALID_ARG, "q_rope_out aliases q_rope_raw");
    }
    if (!ctx_lens) return fail(GQLA_ERR_INVALID_ARG, "ctx_lens is null");
    TRY(check_ptr(latent, "latent"));
    TRY(check_stride(latent_bstride, s.r_kv + s.d_r, max_ctx, "latent_bstride"));
    if (group_cache) {
        TRY(check_ptr(w_uk, "w_uk"));
        TRY(check_ptr(w_uv, "w_uv"));
        TRY(check_ptr(group_cache, "group_cache"));
        TRY(check_stride(group_bstride, 2LL * s.g * s.d_h + s.d_r, max_ctx, "group_bstride"));
    }
    gqla::AppendArgs a;
    a.h_q = s.h_q;
    a.g = s.g;
    a.r_kv = s.r_kv;
    a.d_r = s.d_r;
    a.d_h = s.d_h;
    a.s_q = s.s_q;
    a.batch = batch;
    a.max_ctx = max_ctx;
    a.theta = rope_theta;
    a.c_new = c_new;
    a.kr_new = kr_new;
    a.q_rope_raw = q_rope_raw;
    a.q_rope_out = q_rope_out;
    a.ctx_lens = ctx_lens;
    a.latent = latent;
    a.latent_bstride = latent_bstride;
    a.w_uk = w_uk;
    a.w_uv = w_uv;
    a.group_cache = group_cache;
    a.group_bstride = group_bstride;
    return hip_status(gqla::launch_append(a, s.dtype == GQLA_BF16, static_cast<hipStream_t>(stream)), "append launch");
}

gqla_status gqla_select_path(const gqla_shape* shape, int32_t batch, int64_t total_ctx, double peak_flops,
                             double peak_bytes_per_s, gqla_path_choice* choice) {
    if (!shape) return fail(GQLA_ERR_INVALID_ARG, "shape is null");
    const gqla_shape& s = *shape;
    if (s.h_q <= 0 || s.g <= 0 || s.r_kv <= 0 || s.d_r <= 0 || s.d_h <= 0)
        return fail(GQLA_ERR_INVALID_ARG, "dims must be positive");
    if (s.h_q % s.g != 0) return fail(GQLA_ERR_INVALID_ARG, "h_q=%d is not a multiple of g=%d", s.h_q, s.g);
    if (s.s_q < 1 || s.s_q > 4) return fail(GQLA_ERR_INVALID_ARG, "s_q=%d outside 1..4", s.s_q);
    if (s.dtype != GQLA_BF16 && s.dtype != GQLA_F32) return fail(GQLA_ERR_INVALID_ARG, "unknown dtype %d", s.dtype);
    if (batch < 1 || total_ctx < 1) return fail(GQLA_ERR_INVALID_ARG, "batch and total_ctx must be >= 1");
    if (!(peak_flops > 0.0) || !std::isfinite(peak_flops) || !(peak_bytes_per_s > 0.0) || !std::isfinite(peak_bytes_per_s))
        return fail(GQLA_ERR_INVALID_ARG, "peaks must be finite and > 0");
    if (!choice) return fail(GQLA_ERR_INVALID_ARG, "choice is null");
    const double e = s.dtype == GQLA_BF16 ? 2.0 : 4.0;
    const double T = (double)total_ctx;
    gqla_path_choice best{};
    bool have = false;
    for (int sq = 1; sq <= s.s_q; ++sq) {
        for (int path = GQLA_PATH_ABSORB; path <= GQLA_PATH_GQA; ++path) {
            const double bytes = path == GQLA_PATH_ABSORB ? e * (s.r_kv + s.d_r) : e * (2.0 * s.g * s.d_h + s.d_r);
            const double flops = path == GQLA_PATH_ABSORB ? 2.0 * sq * s.h_q * (2.0 * s.r_kv + s.d_r)
                                                          : 2.0 * sq * s.h_q * (2.0 * s.d_h + s.d_r);
            const double t_mem = bytes * T / peak_bytes_per_s, t_cmp = flops * T / peak_flops;
            const double tps = (double)batch * sq / std::max(t_mem, t_cmp);
            if (!have || tps > best.tokens_per_s) {
                best.path = path;
                best.s_q = sq;
                best.compute_bound = t_cmp > t_mem ? 1 : 0;
                best.reserved = 0;
                best.tokens_per_s = tps;
                have = true;
            }
        }
    }
    *choice = best;
    return ok();
}

gqla_status gqla_measure_peaks(void* scratch, size_t scratch_bytes, double* bytes_per_s, double* flops_per_s,
                               void* stream) {
    constexpr size_t kMin = size_t(64) << 20;
    if (!bytes_per_s || !flops_per_s) return fail(GQLA_ERR_INVALID_ARG, "bytes_per_s or flops_per_s is null");
    TRY(check_ptr(scratch, "scratch"));
    if (scratch_bytes < kMin) return fail(GQLA_ERR_INVALID_ARG, "scratch of %zu bytes < 64 MiB", scratch_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int cus = device_cus();
    TRY(hip_status(gqla::probe_read_bandwidth(scratch, scratch_bytes & ~size_t(15), cus, st, bytes_per_s),
                   "read probe"));
    return hip_status(gqla::probe_mfma_rate(scratch, cus, st, flops_per_s), "mfma probe");
}

gqla_status gqla_set_kernel_events(void* before, void* after) {
    if ((before == nullptr) != (after == nullptr))
        return fail(GQLA_ERR_INVALID_ARG, "set both kernel events or neither");
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
    return ok();
}

const char* gqla_status_string(gqla_status status) {
    switch (status) {
        case GQLA_OK: return "ok";
        case GQLA_ERR_INVALID_ARG: return "invalid argument";
        case GQLA_ERR_UNSUPPORTED: return "unsupported shape";
        case GQLA_ERR_WORKSPACE: return "workspace missing or too small";
        case GQLA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* gqla_last_error(void) { return g_err; }

}  // extern "C"
