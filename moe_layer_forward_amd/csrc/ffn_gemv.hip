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
//  * a persistent grid (a few blocks per CU) walks a list of equal-sized work
//    items, (active expert, chunk of rows); every block compacts the list of
//    active experts of its class from the counts itself, so inactive experts
//    cost nothing and no host round trip or plan kernel is needed;
//  * a wave64 streams whole weight rows with 16-byte coalesced buffer loads
//    (1 KiB per wave instruction).  All loads of one iteration (R rows x MS
//    steps) are issued before any arithmetic: the buffer descriptor's range
//    check returns zeros for out-of-range offsets, so there is no branch
//    between the loads and 16-32 KiB per wave are in flight;
//  * the activation rows of the expert's group (NT tokens per pass) live in
//    VGPRs for the lane's K positions, loaded once and reused for every row;
//  * bf16: one v_dot2_f32_bf16 per weight pair per token, no conversions;
//  * int4-g128: each nibble pair is masked out of the packed dword and XORed
//    with 0x43084308, which flips the nibbles' sign bits (two's complement ->
//    offset binary, q+8) and writes the exponent of bf16 128.0 above them, so
//    each half is exactly the bf16 value 128+q+8; it is dotted with the
//    matching activation pair and 136*sum(x) is subtracted once per 32-element
//    chunk before the fp16 group scale is applied: ~2 VALU ops per weight at
//    2 tokens;
//  * per-lane partials of R rows x NT tokens (x2 for gate/up) are folded with a
//    transposing wave reduction; with KS > 1 the K range is split over KS
//    waves of the block and summed through LDS;
//  * gate/up run in one pass with the SwiGLU epilogue (silu(g)*u) and store h
//    in the activation dtype; the down pass stores fp32 rows of y_perm.
// Experts with c_e == 0 never touch their weights, so the bytes moved are the
// batch union of the selected experts' weights.
#include <type_traits>

#include "common.h"
#include "devinfo.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Transposing reduction of N per-lane values over the 64 lanes of a wave.
// Each of the 6 butterfly levels halves the number of values a lane keeps.
// Afterwards, for N >= 64 lane l holds the totals of values [l*N/64, (l+1)*N/64)
// in v[0..N/64); for N < 64 lane l holds value l >> (6 - log2 N) in v[0].
template <int N>
__device__ __forceinline__ void wave_fold(float (&v)[N], int lane) {
    static_assert(N >= 1 && N <= 256 && (N & (N - 1)) == 0, "N power of two");
    int n = N;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        if (n > 1) {
            // bit masks rather than a select of two array elements: the latter
            // is folded into a lane-dependent array index, which spills to scratch
            const uint32_t m = (lane & o) ? 0xffffffffu : 0u;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                if (i < n / 2) {
                    const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + n / 2]);
                    const uint32_t send = (lo & m) | (hi & ~m);
                    const uint32_t keep = (hi & m) | (lo & ~m);
                    v[i] = __uint_as_float(keep) +
                           __uint_as_float(__builtin_amdgcn_ds_bpermute((lane ^ o) << 2, (int)send));
                }
            }
            n >>= 1;
        } else {
            v[0] += __shfl_xor(v[0], o, MOE_WAVE);
        }
    }
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + nbytes): loads at offsets >= nbytes
// return zero (the hardware range check), which makes masked loads branch-free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                             0x00020000);
}
constexpr uint32_t kOOB = 0xffffffffu;   // an offset the range check always rejects

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2 /* nontemporal */);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
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

// Partial dot product of one 16-byte weight chunk with the first NA of NT
// activation fragments (NA, the tokens present in this pass, is a template
// parameter so the token loops carry no branches).
template <int WT, int ACT, int NT, int NA>
__device__ __forceinline__ void chunk_dot(const uint4& wq, const uint32_t (*xf)[(XDw<WT, ACT>::v)],
                                          const float* xs, float scale, float (&acc)[NT]) {
    const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
    if constexpr (WT == DT_F32) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j >= NA) break;
            float a = acc[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) a = fmaf(__uint_as_float(w[i]), __uint_as_float(xf[j][i]), a);
            acc[j] = a;
        }
    } else if constexpr (WT == DT_BF16) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j >= NA) break;
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
            // nibbles s and s+4 of the dword as the bf16 pair (128 + q + 8): the
            // mask keeps the two nibbles, the XOR flips their sign bit (two's
            // complement -> offset binary) and sets the exponent of 128.0 in
            // the zero bits above them -- one v_bitop3 per pair
            uint32_t m[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) m[s] = ((w[i] >> (4 * s)) & 0x000f000fu) ^ 0x43084308u;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (j >= NA) break;
                float a = part[j];
#pragma unroll
                for (int s = 0; s < 4; ++s) a = dot2_bf16(m[s], xf[j][4 * i + s], a);
                part[j] = a;
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j >= NA) break;
            acc[j] = fmaf(scale, fmaf(-136.0f, xs[j], part[j]), acc[j]);
        }
    }
}

template <int WT, int ACT, int MODE, int NT, int KS, int R, int MS>
__global__ __launch_bounds__(256, 2) void gemv_kernel(GemvArgs a) {
    constexpr int G = (MODE == 0) ? 2 : 1;
    constexpr int EPL = WTraits<WT>::EPL;
    constexpr int DW = XDw<WT, ACT>::v;
    constexpr int RG = 4 / KS;                 // row groups per block
    constexpr int NV = R * G * NT;             // partial sums per lane
    constexpr int PL = NV >= 64 ? NV / 64 : 1; // totals a lane holds after the fold
    constexpr int SH = NV >= 64 ? 0 : (NV == 1 ? 6 : NV == 2 ? 5 : NV == 4 ? 4 : NV == 8 ? 3
                                                : NV == 16 ? 2 : 1);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ks = wave % KS, rg = wave / KS;

    // --- the experts this kernel serves: c_e > 0 and (tau < 0 or c_e <= tau);
    // none when a group of tau < c <= yield_hi rows hands the batch to the
    // skinny kernel
    __shared__ int s_act[256];
    __shared__ int s_wcnt[4], s_wyield[4];
    int U = 1;
    if (a.counts) {
        const int e = threadIdx.x;
        const int c = (e < a.E) ? a.counts[e] : 0;
        const bool act = c > 0 && (a.tau < 0 || c <= a.tau);
        const uint64_t m = __ballot(act);
        const uint64_t y = __ballot(a.yield_hi > 0 && c > a.tau && c <= a.yield_hi);
        if (lane == 0) {
            s_wcnt[wave] = __popcll(m);
            s_wyield[wave] = y != 0ull;
        }
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += s_wcnt[w];
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        if (act) s_act[base + __popcll(m & lt)] = e;
        U = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
        if (s_wyield[0] | s_wyield[1] | s_wyield[2] | s_wyield[3]) U = 0;
        __syncthreads();
    }
    const int nrc = (a.N + a.rows_per_item - 1) / a.rows_per_item;
    const long n_items = (long)U * nrc;
    const long it_begin = n_items * blockIdx.x / gridDim.x;
    const long it_end = n_items * (blockIdx.x + 1) / gridDim.x;

    const int nchunks = a.K / EPL;
    const uint32_t rb = (uint32_t)row_bytes<WT>(a.K);
    const uint32_t mat_bytes = rb * (uint32_t)a.N;
    const uint32_t srow = (uint32_t)(a.K / 128) * 2;     // int4 scale bytes per row
    const size_t in_row = (ACT == DT_F32) ? (size_t)a.K * 4 : (size_t)a.K * 2;
    const size_t out_es = (MODE == 1 || ACT == DT_F32) ? 4 : 2;

    __shared__ float red[2][4][NV];
    int gi = 0;                       // row batches so far: LDS buffer parity
    int cur_e = -1, cur_j0 = -1;      // expert / pass the fragments below belong to
    uint32_t xf[MS][NT][DW];
    float xs[MS][NT];

    for (long item = it_begin; item < it_end; ++item) {
        const int u = (int)(item / nrc);
        const int rc = (int)(item % nrc);
        // wave-uniform by construction; readfirstlane lets the compiler use
        // scalar registers and scalar branches for everything derived from them
        const int e = __builtin_amdgcn_readfirstlane(a.counts ? s_act[u] : 0);
        const int c = __builtin_amdgcn_readfirstlane(a.counts ? a.counts[e] : a.T);
        const int o = __builtin_amdgcn_readfirstlane(a.counts ? a.offsets[e] : 0);
        const int row0 = rc * a.rows_per_item;
        const int row_end = min(a.N, row0 + a.rows_per_item);
        const int niter = (row_end - row0 + RG * R - 1) / (RG * R);

        const char* wb0 = reinterpret_cast<const char*>(a.w0) + (size_t)e * mat_bytes;
        const __amdgpu_buffer_rsrc_t W0 = make_rsrc(wb0, mat_bytes);
        __amdgpu_buffer_rsrc_t W1 = W0, S0 = W0, S1 = W0;
        if constexpr (MODE == 0)
            W1 = make_rsrc(reinterpret_cast<const char*>(a.w1) + (size_t)e * mat_bytes, mat_bytes);
        if constexpr (WT == DT_INT4) {
            S0 = make_rsrc(reinterpret_cast<const char*>(a.s0) + (size_t)e * a.N * srow, a.N * srow);
            if constexpr (MODE == 0)
                S1 = make_rsrc(reinterpret_cast<const char*>(a.s1) + (size_t)e * a.N * srow, a.N * srow);
        }

        for (int j0 = 0; j0 < c; j0 += NT) {
            const int nt = min(NT, c - j0);
            if (e != cur_e || j0 != cur_j0) {
                // activation fragments of this token pass, kept in VGPRs
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const bool tok_ok = j < nt;
                    int src = 0;
                    if (tok_ok) {
                        const int p = o + j0 + j;
                        src = (MODE == 0 && a.perm) ? a.perm[p] / a.topk : p;
                    }
                    const char* rowp = reinterpret_cast<const char*>(a.in) + (size_t)src * in_row;
#pragma unroll
                    for (int s = 0; s < MS; ++s) {
                        const int ch = (s * KS + ks) * 64 + lane;
                        load_x<WT, ACT>(xf[s][j], rowp, ch * EPL, tok_ok && ch < nchunks, &xs[s][j]);
                    }
                }
                cur_e = e;
                cur_j0 = j0;
            }

            // Iteration it+1's loads are issued before iteration it's arithmetic
            // (double-buffered registers): the memory pipe stays busy through the
            // math, the fold and the barrier.  Rows past the item read zeros.
            auto load_iter = [&](int it, uint4 (&wq)[MS][R][G], uint16_t (&sq)[MS][R][G]) {
                const int rbase = row0 + (it * RG + rg) * R;
#pragma unroll
                for (int s = 0; s < MS; ++s) {
                    const int ch = (s * KS + ks) * 64 + lane;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int row = rbase + r;
                        const bool ok = ch < nchunks && row < row_end;
                        const uint32_t off = ok ? (uint32_t)row * rb + (uint32_t)ch * 16u : kOOB;
                        wq[s][r][0] = bload16(W0, off);
                        if constexpr (MODE == 0) wq[s][r][G - 1] = bload16(W1, off);
                        if constexpr (WT == DT_INT4) {
                            const uint32_t so = ok ? (uint32_t)row * srow + (uint32_t)(ch / 4) * 2u : kOOB;
                            sq[s][r][0] = bload2(S0, so);
                            if constexpr (MODE == 0) sq[s][r][G - 1] = bload2(S1, so);
                        }
                    }
                }
            };
            uint4 wqA[MS][R][G], wqB[MS][R][G];
            uint16_t sqA[MS][R][G], sqB[MS][R][G];
            auto body = [&](int it, const uint4 (&wq)[MS][R][G], const uint16_t (&sq)[MS][R][G]) {
                const int rbase = row0 + (it * RG + rg) * R;
                // ---- arithmetic
                float acc[R][G][NT];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int j = 0; j < NT; ++j) acc[r][g][j] = 0.f;
                auto arith = [&](auto na) {
                    constexpr int NA = decltype(na)::value;
#pragma unroll
                    for (int s = 0; s < MS; ++s)
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                const float sc = (WT == DT_INT4) ? f16_to_f32(sq[s][r][g]) : 1.f;
                                chunk_dot<WT, ACT, NT, NA>(wq[s][r][g], xf[s], xs[s], sc, acc[r][g]);
                            }
                };
                // one uniform branch per iteration picks the token count
                switch (nt) {
                    case 1: arith(std::integral_constant<int, 1>{}); break;
                    case 2: if constexpr (NT >= 2) arith(std::integral_constant<int, 2>{}); break;
                    case 3: if constexpr (NT >= 3) arith(std::integral_constant<int, 3>{}); break;
                    case 4: if constexpr (NT >= 4) arith(std::integral_constant<int, 4>{}); break;
                    case 5: if constexpr (NT >= 5) arith(std::integral_constant<int, 5>{}); break;
                    case 6: if constexpr (NT >= 6) arith(std::integral_constant<int, 6>{}); break;
                    case 7: if constexpr (NT >= 7) arith(std::integral_constant<int, 7>{}); break;
                    default: if constexpr (NT >= 8) arith(std::integral_constant<int, 8>{}); break;
                }

                // ---- fold the R*G*NT partials: value v = (r*NT + j)*G + g
                float v[NV];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
#pragma unroll
                        for (int g = 0; g < G; ++g) v[(r * NT + j) * G + g] = acc[r][g][j];
                wave_fold<NV>(v, lane);
                const int vi0 = NV >= 64 ? lane * PL : (lane >> SH);
                const bool writer = NV >= 64 || (lane & ((1 << SH) - 1)) == 0;
                float tot[PL];
#pragma unroll
                for (int i = 0; i < PL; ++i) tot[i] = v[i];
                if constexpr (KS > 1) {
                    float* buf = red[gi & 1][wave];
                    if (writer) {
#pragma unroll
                        for (int i = 0; i < PL; ++i) buf[vi0 + i] = tot[i];
                    }
                    __syncthreads();
                    if (writer) {
#pragma unroll
                        for (int i = 0; i < PL; ++i) {
                            float t = 0.f;
#pragma unroll
                            for (int q = 0; q < KS; ++q) t += red[gi & 1][rg * KS + q][vi0 + i];
                            tot[i] = t;
                        }
                    }
                }
                if (ks != 0) return;
                // ---- epilogue by the ks == 0 wave of each row group
                if constexpr (MODE == 0) {
                    // g has an even value index and u the next one: in the same
                    // lane when a lane holds two or more totals, else 1 << SH lanes up
                    constexpr bool IN_LANE = PL >= 2;
                    float up_v = 0.f;
                    if constexpr (!IN_LANE) up_v = __shfl_down(tot[0], 1 << SH, MOE_WAVE);
                    if (writer) {
#pragma unroll
                        for (int i = 0; i < PL; i += (IN_LANE ? 2 : 1)) {
                            const int vi = vi0 + i;
                            if ((vi & 1) != 0) continue;
                            const float g = tot[i];
                            const float uu = IN_LANE ? tot[(i + 1) % PL] : up_v;
                            const int rj = vi >> 1;
                            const int r = rj / NT, j = rj % NT;
                            const int row = rbase + r;
                            if (row < row_end && j < nt) {
                                const float h = silu(g) * uu;
                                char* op = reinterpret_cast<char*>(a.out) +
                                           ((size_t)(o + j0 + j) * a.N + row) * out_es;
                                if constexpr (ACT == DT_F32) *reinterpret_cast<float*>(op) = h;
                                else *reinterpret_cast<uint16_t*>(op) = f32_to_bf16(h);
                            }
                        }
                    }
                } else {
                    if (writer) {
#pragma unroll
                        for (int i = 0; i < PL; ++i) {
                            const int vi = vi0 + i;
                            const int r = vi / NT, j = vi % NT;
                            const int row = rbase + r;
                            if (row < row_end && j < nt)
                                reinterpret_cast<float*>(a.out)[(size_t)(o + j0 + j) * a.N + row] = tot[i];
                        }
                    }
                }
            };
            load_iter(0, wqA, sqA);
            for (int it = 0; it < niter; it += 2) {
                load_iter(it + 1, wqB, sqB);
                body(it, wqA, sqA);
                ++gi;
                if (it + 1 >= niter) break;
                load_iter(it + 2, wqA, sqA);
                body(it + 1, wqB, sqB);
                ++gi;
            }
        }
    }
}

// ------------------------------------------------------------------ host side

namespace {

struct Variant {
    int ks, ms, nt, r;
};

int epl_of(int wt) { return wt == DT_F32 ? 4 : wt == DT_BF16 ? 8 : 32; }
int dw_of(int wt) { return wt == DT_INT4 ? 16 : 4; }

// Kernel shape for a given K: K split over KS waves, MS 16-byte steps per
// wave, NT tokens per pass, R rows per iteration.  (KS, MS) cover the K steps;
// (NT, R) keep activation fragments + two iterations of weight registers +
// partial sums below 256 VGPRs (no scratch at 2 waves per SIMD) with 8-16
// loads of 16 B in flight per wave.
Variant choose(int wt, int K, int G) {
    const int steps = (K / epl_of(wt) + 63) / 64;
    int ks, ms;
    if (steps <= 1) { ks = 1; ms = 1; }
    else if (steps <= 2) { ks = wt == DT_INT4 ? 2 : 1; ms = wt == DT_INT4 ? 1 : 2; }
    else if (steps <= 4) { ks = wt == DT_INT4 ? 4 : 1; ms = wt == DT_INT4 ? 1 : 4; }
    else if (steps <= 8) { ks = wt == DT_INT4 ? 4 : 2; ms = wt == DT_INT4 ? 2 : 4; }
    else if (steps <= 16) { ks = 4; ms = 4; }
    else if (steps <= 32 && wt != DT_INT4) { ks = 4; ms = 8; }
    else return Variant{0, 0, 0, 0};
    int nt, r;
    const int mi = ms == 1 ? 0 : ms == 2 ? 1 : ms == 4 ? 2 : 3;
    // (NT, R) per MS; the weight registers are double-buffered
    if (wt == DT_INT4) {
        static const int t2[4][2] = {{4, 4}, {4, 1}, {1, 1}, {0, 0}};   // gate/up
        static const int t1[4][2] = {{4, 4}, {4, 2}, {1, 2}, {0, 0}};   // down
        nt = (G == 2 ? t2 : t1)[mi][0];
        r = (G == 2 ? t2 : t1)[mi][1];
    } else {
        static const int t2[4][2] = {{8, 4}, {8, 2}, {8, 1}, {2, 1}};
        static const int t1[4][2] = {{8, 8}, {8, 4}, {8, 2}, {4, 1}};
        nt = (G == 2 ? t2 : t1)[mi][0];
        r = (G == 2 ? t2 : t1)[mi][1];
    }
    return Variant{ks, ms, nt, r};
}

}  // namespace

// Largest K the register-resident activation fragments can hold: 4 waves x
// 8 steps x 64 lanes (bf16, fp32); 4 waves x 4 steps x 64 lanes for int4.
int gemv_max_k(int wt) { return wt == DT_INT4 ? 4 * 4 * 64 * 32 : 4 * 8 * 64 * epl_of(wt); }

template <int WT, int ACT, int MODE, int NT, int KS, int R, int MS>
static hipError_t launch_v(const GemvArgs& a, int max_items, hipStream_t s) {
    auto k = gemv_kernel<WT, ACT, MODE, NT, KS, R, MS>;
    // resident blocks per CU of this variant, per device
    static std::atomic<int> occ[kMaxDevices];
    const int per_cu = per_device_int(occ, [&] {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k, 256, 0) != hipSuccess) v = 1;
        return v;
    });
    const int n_cu = cu_count();
    int grid = per_cu * n_cu;
    if (grid > max_items) grid = max_items;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

#define GEMV_CASE(ks_, ms_, nt_, r_)                                                    \
    if (v.ks == ks_ && v.ms == ms_ && v.nt == nt_ && v.r == r_)                         \
        return launch_v<WT, ACT, MODE, nt_, ks_, r_, ms_>(a, max_items, s);

template <int WT, int ACT, int MODE>
static hipError_t launch_mode(const GemvArgs& a, const Variant& v, int max_items, hipStream_t s) {
    // exactly the (ks, ms, nt, r) tuples choose() returns
    if constexpr (WT == DT_INT4 && MODE == 0) {
        GEMV_CASE(1, 1, 4, 4) GEMV_CASE(2, 1, 4, 4) GEMV_CASE(4, 1, 4, 4)
        GEMV_CASE(4, 2, 4, 1) GEMV_CASE(4, 4, 1, 1)
    } else if constexpr (WT == DT_INT4) {
        GEMV_CASE(1, 1, 4, 4) GEMV_CASE(2, 1, 4, 4) GEMV_CASE(4, 1, 4, 4)
        GEMV_CASE(4, 2, 4, 2) GEMV_CASE(4, 4, 1, 2)
    } else if constexpr (MODE == 0) {
        GEMV_CASE(1, 1, 8, 4) GEMV_CASE(1, 2, 8, 2) GEMV_CASE(1, 4, 8, 1)
        GEMV_CASE(2, 4, 8, 1) GEMV_CASE(4, 4, 8, 1) GEMV_CASE(4, 8, 2, 1)
    } else {
        GEMV_CASE(1, 1, 8, 8) GEMV_CASE(1, 2, 8, 4) GEMV_CASE(1, 4, 8, 2)
        GEMV_CASE(2, 4, 8, 2) GEMV_CASE(4, 4, 8, 2) GEMV_CASE(4, 8, 4, 1)
    }
    return hipErrorInvalidConfiguration;
}
#undef GEMV_CASE

int gemv_pass_tokens(int wt, int mode, int K) { return choose(wt, K, mode == 0 ? 2 : 1).nt; }

hipError_t launch_gemv(int wt, int act, int mode, const GemvArgs& a, int nexp, int max_rows,
                       hipStream_t s) {
    (void)max_rows;
    const Variant v = choose(wt, a.K, mode == 0 ? 2 : 1);
    if (v.nt == 0) return hipErrorInvalidValue;
    const int nrc = (a.N + a.rows_per_item - 1) / a.rows_per_item;
    const int max_items = nexp * nrc;
    if (wt == DT_F32 && act == DT_F32)
        return mode == 0 ? launch_mode<DT_F32, DT_F32, 0>(a, v, max_items, s)
                         : launch_mode<DT_F32, DT_F32, 1>(a, v, max_items, s);
    if (wt == DT_BF16 && act == DT_BF16)
        return mode == 0 ? launch_mode<DT_BF16, DT_BF16, 0>(a, v, max_items, s)
                         : launch_mode<DT_BF16, DT_BF16, 1>(a, v, max_items, s);
    if (wt == DT_INT4 && act == DT_BF16 && i4mfma_supported(a.K, a.N))
        return a.counts ? launch_i4mfma(mode, false, &a, nullptr, s) : launch_i4mfma(mode, false, nullptr, &a, s);
    if (wt == DT_INT4 && act == DT_BF16)
        return mode == 0 ? launch_mode<DT_INT4, DT_BF16, 0>(a, v, max_items, s)
                         : launch_mode<DT_INT4, DT_BF16, 1>(a, v, max_items, s);
    return hipErrorInvalidValue;
}

// Rows of one work item: a multiple of the rows a block covers per iteration,
// sized for about 8 items per block of a 512-block persistent grid (fewer,
// longer items restart the load pipeline less often; enough items keep the
// blocks balanced), at most 64 rows.
int gemv_rows_per_item(int wt, int mode, int K, int N, int active) {
    const Variant v = choose(wt, K, mode == 0 ? 2 : 1);
    const int per_iter = (4 / v.ks) * v.r;
    long want = ((long)active * N + 4095) / 4096;
    if (want > 64) want = 64;
    int rows = per_iter;
    while (rows < want) rows += per_iter;
    return rows;
}

}  // namespace moe
