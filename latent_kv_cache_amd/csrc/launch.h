// Internal interface between the C-ABI host layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqla {

// Everything a decode launch needs, already validated by the host layer.
struct DecodeArgs {
    int h_q, g, r_kv, d_r, d_h, s_q;
    float scale;
    int batch, max_ctx;
    int n_split, chunk;                 // context chunks per sequence, tokens per chunk
    int cus = 0;                        // compute units of the device
    const void* q_nope;
    const void* q_rope;
    const void* w_uk;                   // absorb only
    const void* w_uv;                   // absorb only
    const void* cache;                  // latent rows (absorb) or expanded rows (GQA)
    int64_t bstride;                    // elements between sequences of `cache`
    const int32_t* ctx_lens;
    void* out;
    float* lse;                         // nullable
    float* part_o;                      // [n_split][batch][s_q][h_q][d_h]
    float* part_lse;                    // [n_split][batch][s_q][h_q]
    void* qhat;                         // absorb bf16: [batch][s_q*h_q] absorbed-query records
    void* wpack;                        // absorb bf16: W_UV in the epilogue's operand order
    int n_merge = 0;                    // combine: 0 = the chunks covering L_b, else all n_merge chunks
    hipEvent_t ev_before, ev_after;     // optional, recorded around the main attention kernel
};

inline hipError_t record_if(hipEvent_t ev, hipStream_t st) { return ev ? hipEventRecord(ev, st) : hipSuccess; }

// Blocks of `kernel` (launched with `threads` threads and no dynamic LDS) resident on
// one compute unit at once; 1 if the runtime cannot tell.
template <typename K>
int blocks_per_cu(K kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

struct ExpandArgs {
    int h_q, g, r_kv, d_r, d_h;
    int batch, max_ctx, row_begin;
    const void* latent;
    int64_t latent_bstride;
    const void* w_uk;
    const void* w_uv;
    const int32_t* ctx_lens;
    void* group_cache;
    int64_t group_bstride;
};

// Decode-step append: new latent rows, rotated keys and queries, expanded new rows.
struct AppendArgs {
    int h_q, g, r_kv, d_r, d_h, s_q;
    int batch, max_ctx;
    float theta;
    const void* c_new;                  // [batch][s_q][r_kv]
    const void* kr_new;                 // [batch][s_q][d_r], before rotation
    const void* q_rope_raw;             // [batch][s_q][h_q][d_r] or null
    void* q_rope_out;                   // same shape, or null
    const int32_t* ctx_lens;
    void* latent;
    int64_t latent_bstride;
    const void* w_uk;                   // needed with group_cache
    const void* w_uv;
    void* group_cache;                  // or null
    int64_t group_bstride;
};

hipError_t launch_append(const AppendArgs& a, bool bf16, hipStream_t st);
hipError_t launch_append_fused_bf16(const AppendArgs& a, hipStream_t st);   // rotations and expansion, one launch

// bf16 MFMA path (r_kv = 512, d_r = 64, d_h = 128)
hipError_t launch_absorb_bf16(const DecodeArgs& a, hipStream_t st);
hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t st);
hipError_t launch_expand_bf16(const ExpandArgs& a, hipStream_t st);
bool gqa_bf16_supported(int g, int rows_per_group);
int absorb_block_rows(int query_rows);     // query rows per absorb workgroup (16, 32, 48 or 64)
size_t absorb_qrec_bytes();                // workspace bytes of one absorbed-query record
size_t absorb_wpack_bytes(int g);          // workspace bytes of W_UV in the epilogue's operand order

// sparse GQLA over per-(token, group) index lists (bf16 MFMA or fp32)
hipError_t launch_gqa_sparse(const DecodeArgs& a, const int32_t* indices, int topk, bool bf16, hipStream_t st);

// fp32 vector path (generic dims within the documented bounds)
hipError_t launch_absorb_f32(const DecodeArgs& a, hipStream_t st);
hipError_t launch_gqa_f32(const DecodeArgs& a, hipStream_t st);
// fp32 MFMA kernels, for shapes of whole MFMA tiles (launch_*_f32 pick them when they fit)
bool absorb_f32_mfma_fits(const DecodeArgs& a);
bool gqa_f32_mfma_fits(const DecodeArgs& a);
hipError_t launch_absorb_f32_mfma(const DecodeArgs& a, hipStream_t st);
hipError_t launch_gqa_f32_mfma(const DecodeArgs& a, hipStream_t st);
hipError_t launch_expand_f32(const ExpandArgs& a, hipStream_t st);

// device peak probes (block the host until done)
hipError_t probe_read_bandwidth(const void* buf, size_t bytes, int cus, hipStream_t st, double* bytes_per_s);
hipError_t probe_mfma_rate(void* out, int cus, hipStream_t st, double* flops_per_s);

// split-K log-sum-exp merge of the per-chunk partials into out / lse
hipError_t launch_combine(const DecodeArgs& a, bool out_bf16, hipStream_t st);

// tile sizes the planner must respect
constexpr int kBf16TokenTile = 32;      // chunks are multiples of this on the bf16 path
constexpr int kF32MaxChunk = 1024;      // scores of one chunk live in LDS on the fp32 path

}  // namespace gqla
