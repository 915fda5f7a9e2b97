// Internal launchers of libmoe.so (host side).  Each returns the HIP error of
// its launch; none synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Arguments of the streaming GEMV (ffn_gemv.hip).
struct GemvArgs {
    const void* w0;          // gate (mode 0) or down (mode 1) weights, [E][N][K]
    const void* w1;          // up weights (mode 0), else null
    const uint16_t* s0;      // fp16 group scales of w0 (int4)
    const uint16_t* s1;
    const void* in;          // x [T][K] (mode 0) or h [T*k][K] (mode 1)
    void* out;               // h [T*k][N] (mode 0) or y_perm fp32 [T*k][N] (mode 1)
    const int32_t* counts;   // null: shared expert, all T rows, expert 0
    const int32_t* offsets;
    const int32_t* perm;     // mode 0 only: token = perm[p] / topk
    int N, K, topk, T, E, tau, rows_per_item;
    // > 0: the kernel serves no group at all when some group holds
    // tau < c <= yield_hi rows (the skinny MFMA kernel then takes them all)
    int yield_hi;
};

hipError_t launch_route(int act, const void* x, const float* wg, const float* b, float* logits,
                        int32_t* idx, float* w, int T, int d, int E, int k, hipStream_t s);
struct MfmaPlanArgs;
// plan: when non-null, the dispatch kernel also writes the grouped GEMM's
// tile lists (what launch_mfma_plan would write), saving a launch
hipError_t launch_dispatch(const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, int T, int k, int E, hipStream_t s, const MfmaPlanArgs* plan = nullptr);
// router + softmax + top-k + dispatch of a small decode batch in one kernel
// (T*E within 64 register-held pairs; see route_dispatch_small_supported)
bool route_dispatch_small_supported(int T, int E, int k);
hipError_t launch_route_dispatch_small(int act, const void* x, const float* wg, const float* b, float* logits,
                                       int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int T, int d, int E, int k, hipStream_t s);
// tokens sharing j = 0..k experts between two top-k selections
hipError_t launch_topk_overlap(const int32_t* pred, const int32_t* actual, int32_t* hist, int T, int k,
                               hipStream_t s);
// counts = {n}, offsets = {0, n}, perm = 0..n-1: the shared expert as a group
hipError_t launch_identity_group(int32_t* counts, int32_t* offsets, int32_t* perm, int n, hipStream_t s);
hipError_t launch_gemv(int wt, int act, int mode, const GemvArgs& a, int nexp, int max_rows,
                       hipStream_t s);
int gemv_max_k(int wt);
// Skinny groups of int4-g128, MXFP4 or MXFP8 weights on the matrix cores
// (ffn_i4mfma.hip): K a multiple of 1024 (int4: at most 8192).  One launch serves
// the routed experts (counts/offsets set) and, when `shared` is given, the
// shared expert over all T tokens; either may be null.  `tiled`: 4-bit codes
// (int4 or MXFP4) in the layout launch_pack_int4_tiled writes, or fp8 codes in
// the one launch_pack_mxfp8_tiled writes.  GemvArgs scale pointers
// carry the format's scales (fp16 per 128, or E8M0 bytes per 32).
enum { kFmtInt4 = 0, kFmtFp4 = 1, kFmtFp8 = 2 };
bool i4mfma_supported(int K, int N, int fmt = kFmtInt4);
hipError_t launch_i4mfma(int mode, bool tiled, const GemvArgs* routed, const GemvArgs* shared, hipStream_t s,
                         int fmt = kFmtInt4);
hipError_t launch_pack_int4_tiled(const void* src, void* dst, size_t n_mats, int N, int K, hipStream_t s);
// The same for fp8 codes (MXFP8): two 16-byte pieces per lane and group.
hipError_t launch_pack_mxfp8_tiled(const void* src, void* dst, size_t n_mats, int N, int K, hipStream_t s);
int gemv_rows_per_item(int wt, int mode, int K, int N, int active);
// tokens one GEMV pass holds in registers (a group with more rows streams its
// weights once per pass)
int gemv_pass_tokens(int wt, int mode, int K);
// bf16 groups of up to kSkinnyMaxRows rows on the matrix cores, weights
// streamed once (ffn_skinny.hip): K a multiple of 64.  When the largest
// group of at most `cap` rows holds more than `lo`, every group of 1..cap
// rows is served, else none (the GEMV then serves them).
constexpr int kSkinnyMaxRows = 64;
bool skinny_supported(int K, int N, int in_rows);
hipError_t launch_skinny(int mode, const void* w0, const void* w1, const void* in, int in_rows, void* out,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm, int N, int K,
                         int topk, int E, int lo, int cap, hipStream_t s);
// Quantised expert weights on the matrix cores (ffn_dq.hip): int4 (fmt 0,
// group size gs = 64 or 128, fp16 scales), MXFP4 (1) or MXFP8 (2) with E8M0
// scales per 32; the experts with more than tau rows, in tiles of
// dq_tile_rows(fmt, staged) rows.  staged: the LDS-staged kernel, for passes
// whose K dq_staged_ok accepts (both passes of a layer use the same plan).
int dq_max_tiles(int T, int k, int E);
int dq_plan_ints(int T, int k, int E);
bool dq_supported(int K, int N);
bool dq_staged_ok(int fmt, int gs, int K);
int dq_tile_rows(int fmt, bool staged);
// rem_max > 0: a group's last partial tile of at most rem_max rows is left
// out of the tile list; its rows go to the remainder table dq_remainders()
// (counts [E], then the offsets of those rows [E]; zero elsewhere).
hipError_t launch_dq_plan(const int32_t* counts, const int32_t* offsets, int E, int tau, int fmt, bool staged,
                          int32_t* tiles, int max_mt, int rem_max, hipStream_t s);
int32_t* dq_remainders(int32_t* tiles, int max_mt);
hipError_t launch_dq_ffn(int mode, int fmt, int gs, bool staged, const void* w0, const void* w1, const void* s0,
                         const void* s1, const void* in, void* out, const int32_t* perm, const int32_t* tiles, int N,
                         int K, int topk, int max_mt, int in_rows, hipStream_t s);
int mfma_bm();
int mfma_max_tiles(int T, int k, int E);
int mfma_max_small(int T, int k, int E);
int mfma_plan_ints(int T, int k, int E);
int mfma_ntiles_n(int mode, int N);
// Tile lists of the bf16 grouped GEMM: BOTH puts groups of at most 128 rows
// on 64-row tiles and larger ones on 256-row tiles; SMALL puts every group on
// 64-row tiles and BIG every group on 256-row tiles, and the launch then
// leaves out the kernel whose list is empty.
enum { MFMA_TILES_BOTH = 0, MFMA_TILES_SMALL = 1, MFMA_TILES_BIG = 2 };
constexpr int kMfmaSmallRows = 64;
hipError_t launch_mfma_plan(const int32_t* counts, const int32_t* offsets, int T, int k, int E, int tau,
                            int tile_mode, int32_t* tiles, int max_mt, hipStream_t s);
MfmaPlanArgs mfma_plan_args(int T, int k, int E, int tau, int tile_mode, int32_t* tiles, int max_mt);
hipError_t launch_mfma_ffn(int mode, int tile_mode, const void* w0, const void* w1, const void* in, void* out,
                           const int32_t* perm, const int32_t* tiles, int N, int K, int topk, int T_tokens,
                           int max_mt, int E, int in_rows, float* part, int part_cap, hipStream_t s);
// partial tiles (256 x 256 fp32 each) the split tail round may use
int mfma_part_cap();
hipError_t launch_combine(int act, const float* yp, const int32_t* inv, const float* w,
                          const float* ys, const void* res, void* y, int T, int d, int k,
                          hipStream_t s);
hipError_t launch_rmsnorm(int act, const void* h, const float* gamma, float eps, void* out, int T,
                          int d, hipStream_t s);

}  // namespace moe
