// Expert FFN for prefill-sized groups: a bf16 MFMA grouped GEMM.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §2.1/§3.3: a hand-tiled expert
// GEMM that stages tiles in on-chip shared memory, avoids bank conflicts and
// skips padded rows; experts are grouped so each expert's tokens are
// contiguous ([P2] §2.1, expert-affinity scheduling).
//
// gfx950 design:
//  * a device-side tile plan (one small kernel) turns counts/offsets into a list
//    of 128-row M-tiles, one expert per tile, so no host round trip is needed
//    and idle grid slots exit at once;
//  * 256 threads = 4 wave64s in a 2x2 arrangement own a 128x128 output tile;
//    each wave computes 64x64 with v_mfma_f32_32x32x16_bf16 (fp32 accumulate);
//  * K advances 64 at a time through double-buffered LDS tiles whose rows are
//    padded by 16 bytes so the 16-byte fragment reads of 32 consecutive rows
//    fall in distinct banks; the next K tile is fetched into VGPRs while the
//    current one feeds the MFMAs;
//  * gate and up share the A tile: the B tile holds 64 gate rows then the 64
//    matching up rows, so every lane owns g and u of the same (row, f) and the
//    SwiGLU epilogue needs no data exchange;
//  * A rows of the gate/up GEMM are gathered from x through the permutation
//    (no copy of the dispatched activations is ever made);
//  * grid slots are remapped so consecutive tiles land on one XCD and share
//    its L2.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int MF_BM = 128;
constexpr int MF_BN = 128;
constexpr int MF_BK = 64;
constexpr int MF_LDK = MF_BK + 8;   // padded LDS row, bf16 elements (144 bytes)

int mfma_bm() { return MF_BM; }
int mfma_max_tiles(int T, int k, int E) { return (T * k + MF_BM - 1) / MF_BM + E; }
int mfma_ntiles_n(int mode, int N) { return mode == 0 ? (N + 63) / 64 : (N + MF_BN - 1) / MF_BN; }

__global__ __launch_bounds__(256) void mfma_plan_kernel(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       int tau, int32_t* __restrict__ tiles,
                                                       int max_mt) {
    __shared__ int s[2][256];
    const int tid = threadIdx.x;
    int c = 0, n = 0;
    if (tid < E) {
        c = counts[tid];
        n = (c > tau) ? (c + MF_BM - 1) / MF_BM : 0;
    }
    int cur = 0;
    s[0][tid] = n;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int v = s[cur][tid];
        if (tid >= o) v += s[cur][tid - o];
        s[cur ^ 1][tid] = v;
        cur ^= 1;
        __syncthreads();
    }
    const int start = s[cur][tid] - n;
    if (tid < E) {
        const int o0 = offsets[tid];
        for (int i = 0; i < n; ++i) {
            tiles[start + i] = tid;
            tiles[max_mt + start + i] = o0 + i * MF_BM;
            tiles[2 * max_mt + start + i] = min(MF_BM, c - i * MF_BM);
        }
    }
    if (tid == 255) tiles[3 * max_mt] = s[cur][255];
}

struct MfmaArgs {
    const uint16_t* w0;      // gate (mode 0) or down (mode 1), [E][N][K] bf16
    const uint16_t* w1;      // up (mode 0)
    const uint16_t* in;      // x [T][K] (mode 0) or h [T*k][K] (mode 1), bf16
    void* out;               // h bf16 [T*k][N] (mode 0) or y_perm fp32 [T*k][N] (mode 1)
    const int32_t* perm;
    const int32_t* tiles;    // plan: expert[max_mt], row0[max_mt], rows[max_mt], n_mt
    int N, K, topk, max_mt;
};

template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_ffn_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][MF_BM][MF_LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][MF_BN][MF_LDK];

    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = L % a.max_mt;
    const int nt = L / a.max_mt;
    const int n_mt = a.tiles[3 * a.max_mt];
    if (mt >= n_mt) return;
    const int e = a.tiles[mt];
    const int p0 = a.tiles[a.max_mt + mt];
    const int rows = a.tiles[2 * a.max_mt + mt];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = a.K, N = a.N;

    // global -> LDS assignment: 4 rows per thread (r = tid/8 + 32q), one 16 B column chunk
    const int lrow = tid >> 3, lchunk = tid & 7;
    const uint16_t* arow[4];
    const uint16_t* brow[4];
    const size_t wbase = (size_t)e * N * K;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = lrow + 32 * q;
        const int rr = (r < rows) ? r : 0;
        if (MODE == 0) {
            const int tok = a.perm[p0 + rr] / a.topk;
            arow[q] = a.in + (size_t)tok * K;
        } else {
            arow[q] = a.in + (size_t)(p0 + rr) * K;
        }
        int n;
        const uint16_t* W;
        if (MODE == 0) {
            const int f0 = nt * 64;
            n = f0 + (r & 63);
            W = (r < 64) ? a.w0 : a.w1;
        } else {
            n = nt * MF_BN + r;
            W = a.w0;
        }
        if (n >= N) n = N - 1;
        brow[q] = W + wbase + (size_t)n * K;
    }

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (K + MF_BK - 1) / MF_BK;
    uint4 ra[4], rb[4];
    auto gload = [&](int kt) {
        const int kk = kt * MF_BK + lchunk * 8;
        const bool ok = kk < K;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ra[q] = ok ? *reinterpret_cast<const uint4*>(arow[q] + kk) : make_uint4(0, 0, 0, 0);
            rb[q] = ok ? *reinterpret_cast<const uint4*>(brow[q] + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<uint4*>(&sA[buf][lrow + 32 * q][lchunk * 8]) = ra[q];
            *reinterpret_cast<uint4*>(&sB[buf][lrow + 32 * q][lchunk * 8]) = rb[q];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < MF_BK / 16; ++ks) {
            const int kc = ks * 16 + (lane >> 5) * 8;
            bf16x8_t af[2], bfv[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][wm * 64 + mi * 32 + (lane & 31)][kc]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int br = (MODE == 0) ? (ni * 64 + wn * 32 + (lane & 31)) : (wn * 64 + ni * 32 + (lane & 31));
                bfv[ni] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][br][kc]);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfv[ni], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue; accumulator element v of lane l: column l%32, row 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row >= rows) continue;
            const size_t prow = (size_t)(p0 + row) * N;
            if (MODE == 0) {
                const int f = nt * 64 + wn * 32 + (lane & 31);
                if (f < N) {
                    const float h = silu(acc[mi][0][v]) * acc[mi][1][v];
                    reinterpret_cast<uint16_t*>(a.out)[prow + f] = f32_to_bf16(h);
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int n = nt * MF_BN + wn * 64 + ni * 32 + (lane & 31);
                    if (n < N) reinterpret_cast<float*>(a.out)[prow + n] = acc[mi][ni][v];
                }
            }
        }
    }
}

hipError_t launch_mfma_plan(const int32_t* counts, const int32_t* offsets, int E, int tau,
                            int32_t* tiles, int max_mt, hipStream_t s) {
    hipLaunchKernelGGL(mfma_plan_kernel, dim3(1), dim3(256), 0, s, counts, offsets, E, tau, tiles,
                       max_mt);
    return hipGetLastError();
}

hipError_t launch_mfma_ffn(int mode, const void* w0, const void* w1, const void* in, void* out,
                           const int32_t* perm, const int32_t* tiles, int N, int K, int topk,
                           int max_mt, hipStream_t s) {
    MfmaArgs a;
    a.w0 = reinterpret_cast<const uint16_t*>(w0);
    a.w1 = reinterpret_cast<const uint16_t*>(w1);
    a.in = reinterpret_cast<const uint16_t*>(in);
    a.out = out;
    a.perm = perm;
    a.tiles = tiles;
    a.N = N;
    a.K = K;
    a.topk = topk;
    a.max_mt = max_mt;
    const int grid = max_mt * mfma_ntiles_n(mode, N);
    if (mode == 0)
        hipLaunchKernelGGL(mfma_ffn_kernel<0>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(mfma_ffn_kernel<1>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
