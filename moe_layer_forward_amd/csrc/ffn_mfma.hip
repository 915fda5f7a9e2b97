// Expert FFN for prefill-sized groups: a bf16 MFMA grouped GEMM.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §2.1/§3.3: a hand-tiled expert
// GEMM that stages tiles in on-chip shared memory, avoids bank conflicts and
// skips padded rows; experts are grouped so each expert's tokens are
// contiguous ([P2] §2.1, expert-affinity scheduling).
//
// gfx950 design:
//  * a device-side plan (one small kernel) turns counts/offsets into a list of
//    256-row M-tiles, one expert per tile: no host round trip;
//  * a persistent grid of one 256-thread block per CU walks the (M-tile,
//    N-tile) list.  In every round the 32 CUs of one XCD take 32 consecutive
//    tiles, and tiles are ordered in groups of 8 M-tiles x all N-tiles with M
//    fastest, so concurrent blocks of an XCD share A and B panels in its L2;
//  * block tile 256 x 256; 4 wave64s in a 2x2 arrangement each own
//    128 x 128 = 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (fp32);
//  * LDS holds five stages of A and B of K = 32 each (160 KiB): tiles are
//    copied global -> LDS by buffer_load ... lds (no VGPR staging) two to
//    three K steps ahead of the MFMAs, with one barrier per K step; the copies
//    of two consecutive stages (the two 64-byte halves of each 128-byte row
//    segment) are issued within one step so they meet in the cache.  The
//    lookahead matters more than the pairing: issuing the two halves back to
//    back at the cost of one step of lookahead measured ~20% slower;
//  * the 16-byte chunks of each 64-byte LDS row are XOR-swizzled by
//    (row/4)&3, so 16-byte fragment reads of 16 consecutive rows are
//    conflict-free; each DMA lane simply fetches the chunk that belongs at its
//    fixed LDS slot;
//  * the buffer range check returns zeros for gathered token rows past the
//    group end, weight rows past N and the K tail, so no load is branched;
//  * gate and up share the A tile: the B tile holds 128 gate rows then the 128
//    matching up rows, so each lane owns g and u of the same (row, f) and the
//    SwiGLU epilogue needs no exchange;
//  * A rows of the gate/up GEMM are gathered from x through the permutation;
//    no copy of the dispatched activations is ever made.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int MF_BM = 256;
constexpr int MF_BN = 256;
constexpr int MF_BK = 32;         // K per LDS stage
constexpr int MF_NS = 5;          // LDS stages (2-3 K steps of prefetch in flight)
constexpr int MF_GM = 8;          // M-tiles per scheduling group
constexpr uint32_t MF_OOB = 0x80000000u;   // beyond any buffer: the range check yields 0

constexpr int MS_BM = 64;          // rows of a small M-tile

int mfma_bm() { return MF_BM; }
// Big tiles: experts with more than 128 rows, in 256-row tiles (the tail
// tile's weights stream with the expert's other tiles).  Small tiles: experts
// with at most 128 rows, as one or two 64-row tiles, so a ~50-row group does
// not pay for a 256-row tile.
int mfma_max_tiles(int T, int k, int E) { return (T * k + MF_BM - 1) / MF_BM + E; }
int mfma_max_small(int E) { return 2 * E; }
int mfma_plan_ints(int T, int k, int E) {
    return 3 * mfma_max_tiles(T, k, E) + 1 + 3 * mfma_max_small(E) + 1;
}
int mfma_part_cap() { return 256; }
int mfma_ntiles_n(int mode, int N) { return mode == 0 ? (N + 127) / 128 : (N + MF_BN - 1) / MF_BN; }

// One 256-thread block: per expert with more than tau rows, its big and small
// tiles; exclusive scans over the experts place them.  List layout (ints):
// big: expert[max_mt], row0[max_mt], rows[max_mt], count; then the same for
// the small tiles with max_st entries.
__global__ __launch_bounds__(256) void mfma_plan_kernel(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       int tau, int32_t* __restrict__ tiles,
                                                       int max_mt, int max_st) {
    __shared__ int s[2][2][256];
    const int tid = threadIdx.x;
    int c = 0, nb = 0, ns = 0, rem = 0;
    if (tid < E) {
        c = counts[tid];
        if (c > tau) {
            if (c > 2 * MS_BM) {
                nb = (c + MF_BM - 1) / MF_BM;
            } else {
                rem = c;
                ns = (c + MS_BM - 1) / MS_BM;
            }
        }
    }
    int cur = 0;
    s[0][0][tid] = nb;
    s[0][1][tid] = ns;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int v0 = s[cur][0][tid], v1 = s[cur][1][tid];
        if (tid >= o) { v0 += s[cur][0][tid - o]; v1 += s[cur][1][tid - o]; }
        s[cur ^ 1][0][tid] = v0;
        s[cur ^ 1][1][tid] = v1;
        cur ^= 1;
        __syncthreads();
    }
    int32_t* small = tiles + 3 * max_mt + 1;
    if (tid < E) {
        const int o0 = offsets[tid];
        const int sb = s[cur][0][tid] - nb, ss = s[cur][1][tid] - ns;
        for (int i = 0; i < nb; ++i) {
            tiles[sb + i] = tid;
            tiles[max_mt + sb + i] = o0 + i * MF_BM;
            tiles[2 * max_mt + sb + i] = min(MF_BM, c - i * MF_BM);
        }
        const int base = o0 + c - rem;
        for (int j = 0; j < ns; ++j) {
            small[ss + j] = tid;
            small[max_st + ss + j] = base + j * MS_BM;
            small[2 * max_st + ss + j] = min(MS_BM, rem - j * MS_BM);
        }
    }
    if (tid == 255) {
        tiles[3 * max_mt] = s[cur][0][255];
        small[3 * max_st] = s[cur][1][255];
    }
}

struct MfmaArgs {
    const uint16_t* w0;      // gate (mode 0) or down (mode 1), [E][N][K] bf16
    const uint16_t* w1;      // up (mode 0)
    const uint16_t* in;      // x [T][K] (mode 0) or h [T*k][K] (mode 1), bf16
    void* out;               // h bf16 [T*k][N] (mode 0) or y_perm fp32 [T*k][N] (mode 1)
    const int32_t* perm;
    const int32_t* tiles;    // plan: expert[max_mt], row0[max_mt], rows[max_mt], n_mt
    int N, K, topk, max_mt, max_st, in_rows;
    float* part;             // partial tiles of the split tail round, [part_cap][256][256] fp32
    int part_cap;
};

// The last, partial round of 256-row tiles: W tiles on G blocks leave
// r = W mod G tiles for the final round.  When r <= G/2 each of them is cut
// into S K-ranges (S = G / r, at most the K steps and the partial-buffer
// capacity), so the final round fills the machine; the parts write fp32
// partial tiles, and mfma_tail_reduce sums the S parts of a tile in order.
struct TailSplit {
    int nfull;    // tasks done as whole tiles (R * G)
    int rtail;    // tiles of the last round
    int S;        // parts per tail tile (1: no split)
};
__device__ __forceinline__ TailSplit tail_split(int W, int G, int nk, int cap) {
    TailSplit t;
    const int R = W / G;
    t.rtail = W - R * G;
    t.S = t.rtail > 0 ? G / t.rtail : 1;
    if (t.S > nk) t.S = nk;
    if (t.rtail > 0 && t.rtail * t.S > cap) t.S = cap / t.rtail;
    if (t.S < 2) { t.S = 1; t.nfull = W; t.rtail = 0; }
    else t.nfull = R * G;
    return t;
}


typedef int int32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, 32-bit range, default format) as four dwords.
__device__ __forceinline__ int32x4_t make_desc(const void* base, uint32_t nbytes) {
    const uint64_t b = (uint64_t)base;
    int32x4_t r;   // wave-uniform by construction: keep it in SGPRs
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)nbytes);
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane straight from global memory into LDS: lane l of the wave
// lands at lds_addr + 16*l; an offset the range check rejects writes zeros.
// Issued as inline assembly so that the compiler's wait-count pass does not
// model it: the kernel waits for these copies itself (vmcnt + s_barrier),
// which lets LDS fragment reads of one stage proceed while later stages are
// still being filled.
__device__ __forceinline__ void dma16(const int32x4_t& desc, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(desc), "s"(lds_addr)
                 : "memory");
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)((__attribute__((address_space(3))) const T*)(p)));
}

// wait until at most n (0, 8, 16, 24 or 32) vector-memory operations are outstanding
__device__ __forceinline__ void wait_vm(int n) {
    if (n >= 32) __builtin_amdgcn_s_waitcnt(0x8F70);        // vmcnt(32)
    else if (n >= 24) __builtin_amdgcn_s_waitcnt(0x4F78);   // vmcnt(24)
    else if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);    // vmcnt(8)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
}

__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Swizzled element offset of logical 16-byte chunk `ch` (0..3) of tile row
// `row` in a stage of 32-element (64-byte) rows: four rows share one 256-byte
// bank line and the chunk is XORed with (row/4)&3, so 16 consecutive rows
// reading the same logical chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int ch) {
    return row * MF_BK + ((ch ^ ((row >> 2) & 3)) << 3);
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void mfma_ffn_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[MF_NS][MF_BM * MF_BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[MF_NS][MF_BN * MF_BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = a.K, N = a.N;
    const int n_mt = a.tiles[3 * a.max_mt];
    const int nN = (MODE == 0) ? (N + 127) / 128 : (N + MF_BN - 1) / MF_BN;
    const int total = n_mt * nN;
    const int nblk = gridDim.x;
    // blocks are dealt round-robin to 8 XCDs: give XCD x the slots [x*per, (x+1)*per)
    const int per = nblk / 8;
    const int slot = (nblk % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const int nk = (K + MF_BK - 1) / MF_BK;
    // DMA: each wave instruction fills 16 tile rows x 64 B; this lane owns tile
    // row wave*64 + i*16 + lane/4, physical chunk lane%4
    const int dma_row = wave * 64 + (lane >> 2);
    const int32x4_t RA = make_desc(a.in, (uint32_t)a.in_rows * row_bytes);
    const uint32_t wmat = (uint32_t)N * row_bytes;

    const TailSplit ts = tail_split(total, nblk, nk, a.part_cap);
    const int ntasks = ts.nfull + ts.rtail * ts.S;

    for (int task = slot; task < ntasks; task += nblk) {
        // whole tile, or part s of tail tile j (K steps [kb, ke))
        int L = task, kb = 0, ke = nk, pi = -1;
        if (task >= ts.nfull) {
            const int q = task - ts.nfull, j = q % ts.rtail, sp = q / ts.rtail;
            L = ts.nfull + j;
            kb = (int)((long)nk * sp / ts.S);
            ke = (int)((long)nk * (sp + 1) / ts.S);
            pi = j * ts.S + sp;
        }
        const int kend = min(K, ke * MF_BK);     // element bound of this task's K range
        // grouped order: GM M-tiles x all N-tiles, M fastest
        const int grp = L / (MF_GM * nN);
        const int gm0 = grp * MF_GM;
        const int gsz = min(MF_GM, n_mt - gm0);
        const int rem = L - grp * MF_GM * nN;
        const int mt = gm0 + rem % gsz;
        const int nt = rem / gsz;

        const int e = a.tiles[mt];
        const int p0 = a.tiles[a.max_mt + mt];
        const int rows = a.tiles[2 * a.max_mt + mt];

        // B rows of this wave: mode 0 waves 0-1 hold gate rows, waves 2-3 up rows
        const uint16_t* wsrc = (MODE == 0 && wave >= 2) ? a.w1 : a.w0;
        const int32x4_t RB = make_desc(wsrc + (size_t)e * N * K, wmat);
        uint32_t aoff[4], boff[4];
        int kcol[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = dma_row + i * 16;
            const int ch = (lane & 3) ^ ((r >> 2) & 3);
            kcol[i] = ch * 8;
            if (r < rows) {
                const int src = (MODE == 0) ? a.perm[p0 + r] / a.topk : p0 + r;
                aoff[i] = (uint32_t)src * row_bytes + (uint32_t)ch * 16u;
            } else {
                aoff[i] = MF_OOB;
            }
            const int n = (MODE == 0) ? nt * 128 + (r & 127) : nt * MF_BN + r;
            boff[i] = (n < N) ? (uint32_t)n * row_bytes + (uint32_t)ch * 16u : MF_OOB;
        }
        floatx16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // fragments of one stage: [ks][mi] for A, [ks][ni] for B
        bf16x8_t fa[2][MF_BK / 16][4], fb[2][MF_BK / 16][4];
        auto read_frag = [&](int st, int sl, int q) {   // q: 0..15, A first then B per ks
            const int ks = q >> 3, j = q & 3;
            const int ch = ks * 2 + (lane >> 5);
            if ((q & 4) == 0) {
                fa[sl][ks][j] = *reinterpret_cast<const bf16x8_t*>(
                    &sA[st][swz(wm * 128 + j * 32 + (lane & 31), ch)]);
            } else {
                const int r = (MODE == 0) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32 + (lane & 31))
                                          : (wn * 128 + j * 32 + (lane & 31));
                fb[sl][ks][j] = *reinterpret_cast<const bf16x8_t*>(&sB[st][swz(r, ch)]);
            }
        };
        auto mma = [&](int sl, int m) {                 // m: 0..31 = (ks, mi, ni)
            const int ks = m >> 4, mi = (m >> 2) & 3, ni = m & 3;
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][ks][mi], fb[sl][ks][ni],
                                                                   acc[mi][ni], 0, 0, 0);
        };
        auto issue_one = [&](int kt, int i) {          // DMA i (0..7) of K step kt
            const int st = kt % MF_NS;
            const uint32_t kbyte = (uint32_t)kt * (MF_BK * 2);
            const int k0 = kt * MF_BK;
            const int ii = i >> 1;
            const int r0 = wave * 64 + ii * 16;
            if ((i & 1) == 0) {
                const bool kok = k0 + kcol[ii] < kend;
                dma16(RA, (kok && aoff[ii] != MF_OOB) ? aoff[ii] + kbyte : MF_OOB, lds_addr(&sA[st][r0 * MF_BK]));
            } else {
                const bool kok = k0 + kcol[ii] < kend;
                dma16(RB, (kok && boff[ii] != MF_OOB) ? boff[ii] + kbyte : MF_OOB, lds_addr(&sB[st][r0 * MF_BK]));
            }
        };

        // drain this wave's earlier memory traffic (the previous tile's output
        // stores share the counter) and make sure every wave is done reading
        // the stages before they are refilled
        wait_vm(0);
        block_barrier();
        // Copies of K steps >= nk read out of range and store zeros, so every
        // step below issues exactly 8 copies and the wait counts are constant.
#pragma unroll
        for (int kt = 0; kt < 3; ++kt)
#pragma unroll
            for (int i = 0; i < 8; ++i) issue_one(kb + kt, i);
        wait_vm(16);                 // stage kb landed; kb+1, kb+2 may still fly
        block_barrier();
#pragma unroll
        for (int q = 0; q < 16; ++q) read_frag(kb % MF_NS, 0, q);

        // Software pipeline, per K step kt (fragments of stage kt already in
        // register slot kt&1), with steps taken in pairs from kb:
        //   8 MFMAs | wait: stage kt+1 landed (this wave), own reads done |
        //   barrier | 24 MFMAs interleaved with the 16 reads of stage kt+1 and,
        //   on the first step of a pair, the 16 copies of stages kt+3 and kt+4
        //   (two per third MFMA, all of kt+3 first).  Stages kt+3 and kt+4 hold
        //   the two 64-byte halves of the same 128-byte row segments, so their
        //   copies meet in the cache; the buffers they refill held stages kt-2
        //   and kt-1, which every wave has finished reading.
        //   Outstanding copies at the wait: kt+1, kt+2 on the first step of a
        //   pair (vmcnt 8), kt+2, kt+3, kt+4 on the second (vmcnt 16).
        // The number of steps is rounded up to even: an extra step multiplies
        // zero fragments.
        auto step = [&](int kt, auto slc) {
            constexpr int sl = decltype(slc)::value;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                mma(sl, m);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vm(sl == 0 ? 8 : 16);                     // stage kt+1 landed
            __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): own reads of stage kt done
            block_barrier();
#pragma unroll
            for (int m = 8; m < 32; ++m) {
                mma(sl, m);
                __builtin_amdgcn_sched_barrier(0);
                const int j = m - 8;                       // 0..23
                if (j % 3 == 0) {
                    if constexpr (sl == 0) {
                        const int c = j / 3;               // 0..7: copies 2c, 2c+1
                        const int st = c < 4 ? kt + 3 : kt + 4;
                        issue_one(st, (2 * c) & 7);
                        issue_one(st, (2 * c + 1) & 7);
                    }
                } else {
                    read_frag((kt + 1) % MF_NS, sl ^ 1, j - j / 3 - 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int nk2 = (ke - kb + 1) & ~1;
        for (int kt = kb; kt < kb + nk2; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }

        if (pi >= 0) {
            // a part of a split tail tile: raw fp32 accumulators, tile-local
            // [row][col] with col = the B-tile row the accumulator belongs to
            float* pt = a.part + (size_t)pi * (MF_BM * MF_BN);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 128 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const int col = (MODE == 0) ? (ni >> 1) * 128 + wn * 64 + (ni & 1) * 32 + (lane & 31)
                                                    : wn * 128 + ni * 32 + (lane & 31);
                        pt[row * MF_BN + col] = acc[mi][ni][v];
                    }
                }
            continue;
        }

        // ---- epilogue; accumulator element v of lane l: column l%32, row 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * 128 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row >= rows) continue;
                const size_t prow = (size_t)(p0 + row) * N;
                if (MODE == 0) {
#pragma unroll
                    for (int nj = 0; nj < 2; ++nj) {
                        const int f = nt * 128 + wn * 64 + nj * 32 + (lane & 31);
                        if (f < N) {
                            const float h = silu(acc[mi][nj][v]) * acc[mi][nj + 2][v];
                            reinterpret_cast<uint16_t*>(a.out)[prow + f] = f32_to_bf16(h);
                        }
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const int n = nt * MF_BN + wn * 128 + ni * 32 + (lane & 31);
                        if (n < N) reinterpret_cast<float*>(a.out)[prow + n] = acc[mi][ni][v];
                    }
                }
            }
        }
    }
}

// Sum of the S partial tiles of each split tail tile, in part order, then the
// usual epilogue: y_perm rows (mode 1) or silu(g) * u into h (mode 0).  Block
// (c, j): tail tile j, 1024 outputs (a thread takes 4 consecutive columns of
// one row, reading the S parts with 16-byte loads).
template <int MODE>
__global__ __launch_bounds__(256) void mfma_tail_reduce(MfmaArgs a, int G) {
    const int N = a.N;
    const int n_mt = a.tiles[3 * a.max_mt];
    const int nN = (MODE == 0) ? (N + 127) / 128 : (N + MF_BN - 1) / MF_BN;
    const int nk = (a.K + MF_BK - 1) / MF_BK;
    const TailSplit ts = tail_split(n_mt * nN, G, nk, a.part_cap);
    const int j = blockIdx.y;
    if (j >= ts.rtail) return;
    constexpr int NC = MODE == 0 ? 128 : MF_BN;      // output columns of a tile
    const int idx = (blockIdx.x * 256 + threadIdx.x) * 4;
    const int row = idx / NC, c = idx - row * NC;
    const int L = ts.nfull + j;
    const int grp = L / (MF_GM * nN);
    const int gm0 = grp * MF_GM;
    const int gsz = min(MF_GM, n_mt - gm0);
    const int rem = L - grp * MF_GM * nN;
    const int mt = gm0 + rem % gsz;
    const int nt = rem / gsz;
    const int p0 = a.tiles[a.max_mt + mt];
    const int rows = a.tiles[2 * a.max_mt + mt];
    if (row >= rows) return;
    const float* pt = a.part + (size_t)j * ts.S * (MF_BM * MF_BN) + row * MF_BN + c;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
    for (int sp = 0; sp < ts.S; ++sp) {
        const float4 v = *reinterpret_cast<const float4*>(pt + (size_t)sp * (MF_BM * MF_BN));
        g.x += v.x; g.y += v.y; g.z += v.z; g.w += v.w;
        if (MODE == 0) {
            const float4 w = *reinterpret_cast<const float4*>(pt + (size_t)sp * (MF_BM * MF_BN) + 128);
            u.x += w.x; u.y += w.y; u.z += w.z; u.w += w.w;
        }
    }
    const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
    const size_t orow = (size_t)(p0 + row) * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (MODE == 0) {
            const int f = nt * 128 + c + i;
            if (f < N) reinterpret_cast<uint16_t*>(a.out)[orow + f] = f32_to_bf16(silu(gv[i]) * uv[i]);
        } else {
            const int n = nt * MF_BN + c + i;
            if (n < N) reinterpret_cast<float*>(a.out)[orow + n] = gv[i];
        }
    }
}

// Small M-tiles (at most 64 rows: small expert groups and short remainders).
// Block tile 64 x 256 (gate/up: 128 gate + the 128 matching up rows), four
// waves side by side, each 64 x 64 = 2 x 2 accumulators of
// v_mfma_f32_32x32x16_bf16; K in stages of 32 (4 KiB of A, 16 KiB of B),
// four LDS stages with three stages of copies in flight, 80 KiB of LDS so two
// blocks share a CU.  Such tiles stream each weight tile for few rows, so the
// kernel is bound by the weight stream, not the matrix cores.
constexpr int MS_NS = 4;

template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_small_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[MS_NS][MS_BM * 32];
    __shared__ __attribute__((aligned(16))) uint16_t sB[MS_NS][MF_BN * 32];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int K = a.K, N = a.N;
    const int32_t* tl = a.tiles + 3 * a.max_mt + 1;
    const int max_st = a.max_st;
    const int n_st = tl[3 * max_st];
    const int nN = (MODE == 0) ? (N + 127) / 128 : (N + MF_BN - 1) / MF_BN;
    const int total = n_st * nN;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const int nk = (K + 31) / 32;
    const int32x4_t RA = make_desc(a.in, (uint32_t)a.in_rows * row_bytes);
    const uint32_t wmat = (uint32_t)N * row_bytes;
    // copies: an instruction fills 16 tile rows x 64 B; lane -> row lane/4,
    // physical chunk lane%4.  Wave w copies A rows 16w.. and B rows 64w + 16i..
    const int crow = lane >> 2;

    for (int L = blockIdx.x; L < total; L += gridDim.x) {
        // small tiles of one expert next to each other: consecutive blocks
        // share the weight tile of one N column
        const int st_i = L % n_st, nt = L / n_st;
        const int e = tl[st_i];
        const int p0 = tl[max_st + st_i];
        const int rows = tl[2 * max_st + st_i];

        const uint16_t* wsrc = (MODE == 0 && wave >= 2) ? a.w1 : a.w0;
        const int32x4_t RB = make_desc(wsrc + (size_t)e * N * K, wmat);
        uint32_t aoff, boff[4];
        int acol, bcol[4];
        {
            const int r = wave * 16 + crow;
            const int ch = (lane & 3) ^ ((r >> 2) & 3);
            acol = ch * 8;
            if (r < rows) {
                const int src = (MODE == 0) ? a.perm[p0 + r] / a.topk : p0 + r;
                aoff = (uint32_t)src * row_bytes + (uint32_t)ch * 16u;
            } else {
                aoff = MF_OOB;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 64 + i * 16 + crow;
            const int ch = (lane & 3) ^ ((r >> 2) & 3);
            bcol[i] = ch * 8;
            const int n = (MODE == 0) ? nt * 128 + (r & 127) : nt * MF_BN + r;
            boff[i] = (n < N) ? (uint32_t)n * row_bytes + (uint32_t)ch * 16u : MF_OOB;
        }
        floatx16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        auto issue = [&](int kt) {                     // the 5 copies of this lane for stage kt
            const int st = kt % MS_NS;
            const uint32_t kb = (uint32_t)kt * 64u;
            const int k0 = kt * 32;
            dma16(RA, (k0 + acol < K && aoff != MF_OOB) ? aoff + kb : MF_OOB,
                  lds_addr(&sA[st][(wave * 16) * 32]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dma16(RB, (k0 + bcol[i] < K && boff[i] != MF_OOB) ? boff[i] + kb : MF_OOB,
                      lds_addr(&sB[st][(wave * 64 + i * 16) * 32]));
        };
        auto brow = [&](int ni) {
            return (MODE == 0) ? ni * 128 + wave * 32 + (lane & 31) : wave * 64 + ni * 32 + (lane & 31);
        };
        bf16x8_t fa[2][2][2], fb[2][2][2];            // [slot][ks][mi or ni]
        auto read = [&](int st, int sl) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ch = ks * 2 + (lane >> 5);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    fa[sl][ks][mi] = *reinterpret_cast<const bf16x8_t*>(&sA[st][swz(mi * 32 + (lane & 31), ch)]);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    fb[sl][ks][ni] = *reinterpret_cast<const bf16x8_t*>(&sB[st][swz(brow(ni), ch)]);
            }
        };
        auto mma = [&](int sl) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][ks][mi], fb[sl][ks][ni],
                                                                               acc[mi][ni], 0, 0, 0);
        };

        // previous tile's stores and reads are done before the stages refill
        wait_vm(0);
        block_barrier();
#pragma unroll
        for (int kt = 0; kt < MS_NS; ++kt) issue(kt);  // stages past nk copy zeros
        __builtin_amdgcn_s_waitcnt(0x0F7F);             // vmcnt(15): stage 0 landed
        block_barrier();
        read(0, 0);
        // per stage kt (its fragments in slot kt&1): stage kt+1 landed and every
        // wave is done reading stage kt's buffer -> refill it with stage kt+4,
        // read stage kt+1, multiply stage kt
        auto step = [&](int kt, auto slc) {
            constexpr int sl = decltype(slc)::value;
            __builtin_amdgcn_s_waitcnt(0x0F7A);         // vmcnt(10): stage kt+1 landed
            __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): own reads of stage kt done
            block_barrier();
            issue(kt + MS_NS);
            read((kt + 1) % MS_NS, sl ^ 1);
            mma(sl);
        };
        const int nk2 = (nk + 1) & ~1;                  // an extra step multiplies zeros
        for (int kt = 0; kt < nk2; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }

        // ---- epilogue; accumulator element v of lane l: column l%32, row 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row >= rows) continue;
                const size_t prow = (size_t)(p0 + row) * N;
                if (MODE == 0) {
                    const int f = nt * 128 + wave * 32 + (lane & 31);
                    if (f < N) {
                        const float h = silu(acc[mi][0][v]) * acc[mi][1][v];
                        reinterpret_cast<uint16_t*>(a.out)[prow + f] = f32_to_bf16(h);
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const int n = nt * MF_BN + wave * 64 + ni * 32 + (lane & 31);
                        if (n < N) reinterpret_cast<float*>(a.out)[prow + n] = acc[mi][ni][v];
                    }
                }
            }
        }
    }
}

hipError_t launch_mfma_plan(const int32_t* counts, const int32_t* offsets, int E, int tau,
                            int32_t* tiles, int max_mt, hipStream_t s) {
    hipLaunchKernelGGL(mfma_plan_kernel, dim3(1), dim3(256), 0, s, counts, offsets, E, tau, tiles,
                       max_mt, mfma_max_small(E));
    return hipGetLastError();
}

hipError_t launch_mfma_ffn(int mode, const void* w0, const void* w1, const void* in, void* out,
                           const int32_t* perm, const int32_t* tiles, int N, int K, int topk,
                           int max_mt, int E, int in_rows, float* part, int part_cap, hipStream_t s) {
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
    a.max_st = mfma_max_small(E);
    a.in_rows = in_rows;
    a.part = part;
    a.part_cap = part ? part_cap : 0;
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
            n_cu = 256;
    }
    const int nN = mfma_ntiles_n(mode, N);
    // big tiles: one 256-thread block per CU
    const int slots = max_mt * nN;
    const int grid = slots < n_cu ? slots : n_cu;
    if (mode == 0)
        hipLaunchKernelGGL(mfma_ffn_kernel<0>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(mfma_ffn_kernel<1>, dim3(grid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.part_cap > 0) {
        // sums of the split tail tiles (blocks without such a tile exit at once)
        if (mode == 0)
            hipLaunchKernelGGL(mfma_tail_reduce<0>, dim3(MF_BM * 128 / 1024, grid), dim3(256), 0, s, a, grid);
        else
            hipLaunchKernelGGL(mfma_tail_reduce<1>, dim3(MF_BM * MF_BN / 1024, grid), dim3(256), 0, s, a, grid);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // small tiles: two blocks per CU
    const int sslots = a.max_st * nN;
    const int sgrid = sslots < 2 * n_cu ? sslots : 2 * n_cu;
    if (mode == 0)
        hipLaunchKernelGGL(mfma_small_kernel<0>, dim3(sgrid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(mfma_small_kernel<1>, dim3(sgrid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
