// Expert FFN for decode-sized groups: an HBM-streaming GEMV.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §3.3: each expert's kernel
// receives the token map and the expert offsets and streams that expert's
// weights; small-M x large-N x K is the shape of the problem (§2.1).  [P3]
// (wzjinhao.cn) §2.3: only active experts run.  The pages' A100 kernel tiles
// through shared memory; at decode the work is bandwidth-bound (every weight
// byte is used by ~2 rows), so here nothing is staged in LDS at all.
//
// gfx950 design:
//  * a wave64 streams whole weight rows with 16-byte coalesced loads (1 KiB per
//    wave instruction), R rows at a time so that many bytes are in flight;
//  * the activation rows of the expert's group (NT tokens per pass) live in
//    VGPRs for the lane's K positions, loaded once and reused for every row;
//  * bf16: one v_dot2_f32_bf16 per weight pair per token, no conversions;
//  * int4-g128: codes are XORed with 0x8 (two's complement -> offset binary),
//    each nibble pair is OR-ed into the mantissa of bf16 128.0 (0x4300|u is
//    exactly 128+u), dotted with the matching activation pair, and the constant
//    136*sum(x) is subtracted once per 32-element chunk before the fp16 group
//    scale is applied: ~2 VALU ops per weight at 2 tokens;
//  * per-lane partials of R rows x NT tokens (x2 for gate/up) are folded with a
//    transposing wave reduction; with KS > 1 the K range is split over KS
//    waves of the block and summed through LDS;
//  * gate/up run in one pass with the SwiGLU epilogue (silu(g)*u) and store h
//    in the activation dtype; the down pass stores fp32 rows of y_perm.
// Experts with c_e == 0 never touch their weights, so the bytes moved are the
// batch union of the selected experts' weights.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int N>
__device__ __forceinline__ void wave_fold(float (&v)[N], int lane) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N power of two");
    int n = N;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        if (n > 1) {
            const bool up = (lane & o) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                if (i < n / 2) {
                    float send = up ? v[i] : v[i + n / 2];
                    float keep = up ? v[i + n / 2] : v[i];
                    v[i] = keep + __shfl_xor(send, o, MOE_WAVE);
                }
            }
            n >>= 1;
        } else {
            v[0] += __shfl_xor(v[0], o, MOE_WAVE);
        }
    }
}

template <int WT> struct WTraits;
template <> struct WTraits<DT_F32> { static constexpr int EPL = 4; };    // 16 B = 4 fp32
template <> struct WTraits<DT_BF16> { static constexpr int EPL = 8; };   // 16 B = 8 bf16
template <> struct WTraits<DT_INT4> { static constexpr int EPL = 32; };  // 16 B = 32 int4

// activation dwords per lane per step
template <int WT, int ACT> struct XDw {
    static constexpr int v = (ACT == DT_F32) ? WTraits<WT>::EPL : WTraits<WT>::EPL / 2;
};

template <int WT>
__device__ __forceinline__ size_t row_bytes(int K) {
    if constexpr (WT == DT_F32) return (size_t)K * 4;
    else if constexpr (WT == DT_BF16) return (size_t)K * 2;
    else return (size_t)K / 2;
}

// Load the lane's activation fragment of one step (EPL elements at kk).
template <int WT, int ACT>
__device__ __forceinline__ void load_x(uint32_t (&dst)[(XDw<WT, ACT>::v)], const void* row, int kk,
                                       bool ok, float* xsum) {
    constexpr int DW = XDw<WT, ACT>::v;
    if (!ok) {
#pragma unroll
        for (int i = 0; i < DW; ++i) dst[i] = 0u;
        if (xsum) *xsum = 0.f;
        return;
    }
    if constexpr (ACT == DT_F32) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(row) + kk);
#pragma unroll
        for (int i = 0; i < DW / 4; ++i) {
            uint4 q = p[i];
            dst[4 * i] = q.x; dst[4 * i + 1] = q.y; dst[4 * i + 2] = q.z; dst[4 * i + 3] = q.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(row) + kk);
        uint32_t raw[DW];
#pragma unroll
        for (int i = 0; i < DW / 4; ++i) {
            uint4 q = p[i];
            raw[4 * i] = q.x; raw[4 * i + 1] = q.y; raw[4 * i + 2] = q.z; raw[4 * i + 3] = q.w;
        }
        if constexpr (WT == DT_INT4) {
            // Pair element k+s with k+s+4 inside each group of 8 (one weight dword):
            // dword s of the group = (x[k+s] lo, x[k+s+4] hi).
            float sum = 0.f;
#pragma unroll
            for (int g = 0; g < DW / 4; ++g) {
                const uint32_t a = raw[4 * g], b = raw[4 * g + 1], c = raw[4 * g + 2], d = raw[4 * g + 3];
                // elements: a=(0,1) b=(2,3) c=(4,5) d=(6,7)
                dst[4 * g + 0] = (a & 0xffffu) | (c << 16);          // (0,4)
                dst[4 * g + 1] = (a >> 16) | (c & 0xffff0000u);      // (1,5)
                dst[4 * g + 2] = (b & 0xffffu) | (d << 16);          // (2,6)
                dst[4 * g + 3] = (b >> 16) | (d & 0xffff0000u);      // (3,7)
                sum += bf16_lo(a) + bf16_hi(a) + bf16_lo(b) + bf16_hi(b) + bf16_lo(c) + bf16_hi(c) +
                       bf16_lo(d) + bf16_hi(d);
            }
            *xsum = sum;
        } else {
#pragma unroll
            for (int i = 0; i < DW; ++i) dst[i] = raw[i];
        }
    }
}

// Partial dot product of one 16-byte weight chunk with NT activation fragments.
template <int WT, int ACT, int NT>
__device__ __forceinline__ void chunk_dot(const uint4& wq, const uint32_t (*xf)[(XDw<WT, ACT>::v)],
                                          const float* xs, float scale, float (&acc)[NT]) {
    const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
    if constexpr (WT == DT_F32) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float a = acc[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) a = fmaf(__uint_as_float(w[i]), __uint_as_float(xf[j][i]), a);
            acc[j] = a;
        }
    } else if constexpr (WT == DT_BF16) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float a = acc[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) a = dot2_bf16(w[i], xf[j][i], a);
            acc[j] = a;
        }
    } else {
        // 4 dwords x 8 nibbles; dword i covers elements 8i..8i+7
        float part[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) part[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = w[i] ^ 0x88888888u;   // q + 8 in every nibble
            uint32_t m[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) m[s] = ((u >> (4 * s)) & 0x000f000fu) | 0x43004300u;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                float a = part[j];
#pragma unroll
                for (int s = 0; s < 4; ++s) a = dot2_bf16(m[s], xf[j][4 * i + s], a);
                part[j] = a;
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = fmaf(scale, fmaf(-136.0f, xs[j], part[j]), acc[j]);
    }
}

template <int WT, int ACT, int MODE, int NT, int KS, int R, int MS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    constexpr int G = (MODE == 0) ? 2 : 1;
    constexpr int EPL = WTraits<WT>::EPL;
    constexpr int DW = XDw<WT, ACT>::v;
    constexpr int RG = 4 / KS;                 // row groups per block
    constexpr int NV = R * G * NT;             // partial sums per lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ks = wave % KS, rg = wave / KS;
    const int e = blockIdx.y;

    int c, o;
    if (a.counts) {
        c = a.counts[e];
        o = a.offsets[e];
        if (c == 0 || (a.tau >= 0 && c > a.tau)) return;
    } else {
        c = a.T;
        o = 0;
        if (c == 0) return;
    }
    const int row0 = blockIdx.x * a.rows_per_block;
    const int row_end = min(a.N, row0 + a.rows_per_block);
    if (row0 >= row_end) return;

    const int nchunks = a.K / EPL;
    const int nsteps = (nchunks + 63) / 64;
    const size_t rb = row_bytes<WT>(a.K);
    const char* W0 = reinterpret_cast<const char*>(a.w0) + (size_t)e * a.N * rb;
    const char* W1 = (MODE == 0) ? reinterpret_cast<const char*>(a.w1) + (size_t)e * a.N * rb : nullptr;
    const uint16_t* S0 = (WT == DT_INT4) ? a.s0 + (size_t)e * a.N * (a.K / 128) : nullptr;
    const uint16_t* S1 = (WT == DT_INT4 && MODE == 0) ? a.s1 + (size_t)e * a.N * (a.K / 128) : nullptr;
    const size_t in_row = (ACT == DT_F32) ? (size_t)a.K * 4 : (size_t)a.K * 2;
    const size_t out_es = (MODE == 1 || ACT == DT_F32) ? 4 : 2;

    __shared__ float red[2][4][NV];
    const int niter = (row_end - row0 + RG * R - 1) / (RG * R);
    int gi = 0;   // row batches done so far: selects the LDS buffer (parity spans passes)

    for (int j0 = 0; j0 < c; j0 += NT) {
        // activation fragments of this token pass, kept in VGPRs
        uint32_t xf[MS][NT][DW];
        float xs[MS][NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const bool tok_ok = j0 + j < c;
            int src = 0;
            if (tok_ok) {
                const int p = o + j0 + j;
                src = (MODE == 0 && a.perm) ? a.perm[p] / a.topk : p;
            }
            const char* rowp = reinterpret_cast<const char*>(a.in) + (size_t)src * in_row;
#pragma unroll
            for (int s = 0; s < MS; ++s) {
                const int gs = s * KS + ks;
                const int ch = gs * 64 + lane;
                load_x<WT, ACT>(xf[s][j], rowp, ch * EPL, tok_ok && gs < nsteps && ch < nchunks,
                                &xs[s][j]);
            }
        }

        for (int it = 0; it < niter; ++it, ++gi) {
            const int rbase = row0 + (it * RG + rg) * R;
            float acc[R][G][NT];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[r][g][j] = 0.f;

#pragma unroll
            for (int s = 0; s < MS; ++s) {
                const int gs = s * KS + ks;
                if (gs >= nsteps) break;
                const int ch = gs * 64 + lane;
                const bool kok = ch < nchunks;
                uint4 wq[R][G];
                float sc[R][G];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = rbase + r;
                    const bool ok = kok && row < row_end;
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const char* Wm = (g == 0) ? W0 : W1;
                        wq[r][g] = ok ? *reinterpret_cast<const uint4*>(Wm + (size_t)row * rb + (size_t)ch * 16)
                                      : make_uint4(0u, 0u, 0u, 0u);
                        if constexpr (WT == DT_INT4) {
                            const uint16_t* Sm = (g == 0) ? S0 : S1;
                            sc[r][g] = ok ? f16_to_f32(Sm[(size_t)row * (a.K / 128) + (ch * EPL) / 128]) : 0.f;
                        } else {
                            sc[r][g] = 1.f;
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        chunk_dot<WT, ACT, NT>(wq[r][g], xf[s], xs[s], sc[r][g], acc[r][g]);
            }

            // fold the R*G*NT partials across the wave: value v = (r*NT + j)*G + g
            float v[NV];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int g = 0; g < G; ++g) v[(r * NT + j) * G + g] = acc[r][g][j];
            wave_fold<NV>(v, lane);
            constexpr int SH = (NV == 1) ? 6 : (NV == 2) ? 5 : (NV == 4) ? 4 : (NV == 8) ? 3
                             : (NV == 16) ? 2 : (NV == 32) ? 1 : 0;
            const int vi = lane >> SH;               // value index this lane holds
            const bool writer = (lane & ((1 << SH) - 1)) == 0;
            float total;
            if constexpr (KS == 1) {
                total = v[0];
            } else {
                float* buf = red[gi & 1][wave];
                if (writer) buf[vi] = v[0];
                __syncthreads();
                total = 0.f;
                if (writer) {
#pragma unroll
                    for (int q = 0; q < KS; ++q) total += red[gi & 1][rg * KS + q][vi];
                }
            }
            // epilogue by the ks == 0 wave of each row group
            if (ks == 0) {
                if constexpr (MODE == 0) {
                    // g at even value index, u at the next one (1 << SH lanes above)
                    const float u = __shfl_down(total, 1 << SH, MOE_WAVE);
                    if (writer && (vi & 1) == 0) {
                        const int rj = vi >> 1;
                        const int r = rj / NT, j = rj % NT;
                        const int row = rbase + r;
                        if (row < row_end && j0 + j < c) {
                            const float h = silu(total) * u;
                            char* op = reinterpret_cast<char*>(a.out) +
                                       ((size_t)(o + j0 + j) * a.N + row) * out_es;
                            if constexpr (ACT == DT_F32) *reinterpret_cast<float*>(op) = h;
                            else *reinterpret_cast<uint16_t*>(op) = f32_to_bf16(h);
                        }
                    }
                } else {
                    if (writer) {
                        const int r = vi / NT, j = vi % NT;
                        const int row = rbase + r;
                        if (row < row_end && j0 + j < c)
                            reinterpret_cast<float*>(a.out)[(size_t)(o + j0 + j) * a.N + row] = total;
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ host side

template <int WT, int ACT, int MODE, int NT, int KS>
static hipError_t launch_one(const GemvArgs& a, int nexp, hipStream_t s) {
    constexpr int R = (WT == DT_INT4) ? 2 : 2;
    constexpr int MS = (WT == DT_INT4) ? 4 : 8;
    dim3 grid((a.N + a.rows_per_block - 1) / a.rows_per_block, nexp);
    hipLaunchKernelGGL((gemv_kernel<WT, ACT, MODE, NT, KS, R, MS>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int WT, int ACT, int MODE, int NT>
static hipError_t launch_ks(const GemvArgs& a, int nexp, int ks, hipStream_t s) {
    if (ks == 1) return launch_one<WT, ACT, MODE, NT, 1>(a, nexp, s);
    return launch_one<WT, ACT, MODE, NT, 4>(a, nexp, s);
}

template <int WT, int ACT, int MODE>
static hipError_t launch_nt(const GemvArgs& a, int nexp, int ks, int nt, hipStream_t s) {
    if (nt <= 1) return launch_ks<WT, ACT, MODE, 1>(a, nexp, ks, s);
    if (nt <= 2) return launch_ks<WT, ACT, MODE, 2>(a, nexp, ks, s);
    return launch_ks<WT, ACT, MODE, 4>(a, nexp, ks, s);
}

int gemv_max_steps(int wt) { return wt == DT_INT4 ? 4 : 8; }
int gemv_epl(int wt) { return wt == DT_F32 ? 4 : wt == DT_BF16 ? 8 : 32; }

// Largest K the register-resident activation fragments can hold.
int gemv_max_k(int wt) { return gemv_max_steps(wt) * 4 * 64 * gemv_epl(wt); }

static int choose_ks(int wt, int K) {
    const int nsteps = (K / gemv_epl(wt) + 63) / 64;
    return nsteps <= gemv_max_steps(wt) ? 1 : 4;
}

static int choose_nt(int wt, int max_rows) {
    const int cap = (wt == DT_INT4) ? 2 : 4;
    int nt = 1;
    while (nt < cap && nt < max_rows) nt *= 2;
    return nt;
}

hipError_t launch_gemv(int wt, int act, int mode, const GemvArgs& a, int nexp, int max_rows,
                       hipStream_t s) {
    const int ks = choose_ks(wt, a.K);
    const int nt = choose_nt(wt, max_rows);
    if (wt == DT_F32 && act == DT_F32) {
        return mode == 0 ? launch_nt<DT_F32, DT_F32, 0>(a, nexp, ks, nt, s)
                         : launch_nt<DT_F32, DT_F32, 1>(a, nexp, ks, nt, s);
    }
    if (wt == DT_BF16 && act == DT_BF16) {
        return mode == 0 ? launch_nt<DT_BF16, DT_BF16, 0>(a, nexp, ks, nt, s)
                         : launch_nt<DT_BF16, DT_BF16, 1>(a, nexp, ks, nt, s);
    }
    if (wt == DT_INT4 && act == DT_BF16) {
        return mode == 0 ? launch_nt<DT_INT4, DT_BF16, 0>(a, nexp, ks, nt, s)
                         : launch_nt<DT_INT4, DT_BF16, 1>(a, nexp, ks, nt, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
