// Expert FFN for prefill-sized groups: a bf16 MFMA grouped GEMM.
//
// [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" §2.1/§3.3: a hand-tiled expert
// GEMM that stages tiles in on-chip shared memory, avoids bank conflicts and
// skips padded rows; experts are grouped so each expert's tokens are
// contiguous ([P2] §2.1, expert-affinity scheduling).
//
// gfx950 design:
//  * a device-side plan (one wave, plan.h: at the end of the dispatch kernel
//    inside the layer call, else its own launch) turns counts/offsets into a
//    list of 256-row M-tiles, one expert per tile: no host round trip;
//  * a persistent grid of one 512-thread block per CU walks the (M-tile,
//    N-tile) list.  In every round the 32 CUs of one XCD take 32 consecutive
//    tiles, and tiles are ordered in groups of 8 M-tiles x all N-tiles with M
//    fastest, so concurrent blocks of an XCD share A and B panels in its L2;
//  * block tile 256 x 256, eight wave64s in two groups of four (waves i and
//    i+4 share a SIMD).  The groups ping-pong: while one issues the 16 MFMAs
//    of a K step (v_mfma_f32_32x32x16_bf16, fp32 accumulators), the other
//    reads its fragments of the step from LDS; a block barrier swaps the
//    roles.  With K a multiple of 64 the global -> LDS copies go out between
//    the MFMAs of the compute phase (each copy holds its wave ~60-75 cycles at
//    issue, which the memory phase cannot spare, while an MFMA leaves room
//    for one), their offsets worked out in the memory phase before; other K
//    issue them at the end of the memory phase.  Group g owns tile rows
//    128g..128g+127; wave i of a group owns 64 B-tile rows (4 x 2
//    accumulators);
//  * the product is computed transposed (weights as the MFMA A operand), so a
//    lane's accumulator holds four consecutive output columns of one token
//    row: the epilogue stores 16 (fp32) or 8 (bf16) bytes per lane straight
//    from registers, no LDS round trip;
//  * LDS holds K in pairs of steps (K = 64, one 128-byte row per tile row):
//    two A pair slots and three B pair slots (160 KiB), refilled by
//    buffer_load ... lds (no VGPR staging).  Every copy instruction moves 8
//    rows x one whole 128-byte line; copies of 16 rows x 64 B (one K step per
//    slot) cost the texture path ~10% of the GEMM.  Step 2j issues the next A
//    pair, step 2j+1 the B pair after next, four copies per wave per step,
//    each landing two or more steps before its first read.  The copy stream
//    runs on across the block's tiles: a tile's last pairs fetch the next
//    tile's first ones, so no tile starts on an empty pipeline;
//  * the 16-byte chunks of each 128-byte LDS row are XOR-swizzled by
//    (row/2)&7, so 16-byte fragment reads of 16 consecutive rows are
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
#include "devinfo.h"
#include "kernels.h"
#include "lds_dma.h"
#include "plan.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int MF_BM = kMfmaBigRows;
constexpr int MF_BN = 256;
constexpr int MF_BK = 32;         // K per LDS stage
constexpr int MF_GM = 8;          // M-tiles per scheduling group
constexpr uint32_t MF_OOB = 0x80000000u;   // beyond any buffer: the range check yields 0
constexpr int kNonTemporal = 2;            // buffer-load cache policy: streamed, not kept

constexpr int MS_BM = kMfmaSmallRows;   // rows of a small M-tile

template <int I>
using ic = std::integral_constant<int, I>;
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

int mfma_bm() { return MF_BM; }
// Big tiles: experts with more than 128 rows, in 256-row tiles (the tail
// tile's weights stream with the expert's other tiles).  Small tiles: experts
// with at most 128 rows, as one or two 64-row tiles, so a ~50-row group does
// not pay for a 256-row tile.  With one list only (MFMA_TILES_SMALL / _BIG)
// every group goes to that list; the bounds hold for any split of T*k rows
// over E experts.
int mfma_max_tiles(int T, int k, int E) { return (T * k + MF_BM - 1) / MF_BM + E; }
int mfma_max_small(int T, int k, int E) { return (T * k + MS_BM - 1) / MS_BM + E; }
int mfma_plan_ints(int T, int k, int E) {
    return 3 * mfma_max_tiles(T, k, E) + 1 + 3 * mfma_max_small(T, k, E) + 1;
}
int mfma_part_cap() { return 256; }
int mfma_ntiles_n(int mode, int N) { return mode == 0 ? (N + 127) / 128 : (N + MF_BN - 1) / MF_BN; }

// The tile lists (plan.h) from counts and offsets: one wave.
__global__ __launch_bounds__(64) void mfma_plan_kernel(const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      MfmaPlanArgs p) {
    const int lane = threadIdx.x;
    int c[4], o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        c[j] = e < E ? counts[e] : 0;
        o[j] = e < E ? offsets[e] : 0;
    }
    mfma_plan_wave(lane, c, o, E, p);
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
// into S K-ranges (S = G / r, at most the K pairs and the partial-buffer
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


// Pair slots of the 256-row kernel: K = 64 (two K steps) per 128-byte LDS row,
// so that every copy instruction moves whole 128-byte lines (8 rows x 128 B).
// The 16-byte chunks of a row are XORed with (row/2)&7: rows 2j and 2j+1 share
// a 256-byte bank line, and 16 consecutive rows reading the same logical chunk
// land on 16 distinct 16-byte bank groups.
constexpr int MF_PK = 2 * MF_BK;              // K per pair slot
constexpr int MF_PSLOT = MF_BM * MF_PK;       // elements of one operand pair slot
constexpr int MF_AS = 2;                      // A pair slots
constexpr int MF_BS = 3;                      // B pair slots
__device__ __forceinline__ int swz2(int row, int ch) {
    return row * MF_PK + ((ch ^ ((row >> 1) & 7)) << 3);
}

// wait until at most n (0, 4, 8 or 12) vector-memory operations are outstanding
__device__ __forceinline__ void wait_copies(int n) {
    if (n >= 12) __builtin_amdgcn_s_waitcnt(0x0F7C);        // vmcnt(12)
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);    // vmcnt(8)
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);    // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
}

// FAST (K a multiple of 64, at least two K pairs): every copy is issued from
// the compute phase, between the MFMAs, with its offsets worked out during the
// memory phase before; the memory phase then holds only the fragment reads.
// Otherwise the copies go out in the memory phase (K tails, single pairs).
// Task L of the grouped order -> (M-tile, N-tile): groups of MF_GM M-tiles x
// all N-tiles, M fastest.  Within a group the M position turns by one every
// 32 N-tiles (one round of a 256-block grid: 256 tasks), so a block does not
// keep the same M position -- say an expert's ragged last tile -- round after
// round; the 32 tasks an XCD takes in a round still span MF_GM M-tiles and
// 4 N-tiles.
__device__ __forceinline__ void grouped_tile(int L, int n_mt, int nN, int& mt, int& nt) {
    const int grp = L / (MF_GM * nN);
    const int gm0 = grp * MF_GM;
    const int gsz = min(MF_GM, n_mt - gm0);
    const int rem = L - grp * MF_GM * nN;
    nt = rem / gsz;
    mt = gm0 + (rem % gsz + (nt >> 5)) % gsz;
}

template <int MODE, bool FAST>
__global__ __launch_bounds__(512, 1) void mfma_ffn_kernel(MfmaArgs a) {
    // A pair slots then B pair slots; pair j of a task (its K steps kb + 2j and
    // kb + 2j + 1) sits in A slot j % 2 and B slot j % 3
    __shared__ __attribute__((aligned(16))) uint16_t smem[(MF_AS + MF_BS) * MF_PSLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wi = wave & 3;
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
    const int np = (nk + 1) / 2;                 // K pairs
    // copies: wave w fills A rows and B rows 32w + 8i + lane/8 (i = 0..3),
    // physical chunk lane%8 of the 128-byte row
    const int32x4_t RA = make_desc(a.in, (uint32_t)a.in_rows * row_bytes);
    const uint32_t wmat = (uint32_t)N * row_bytes;
    // B rows of this wave's copies: mode 0 waves 0-3 gate rows, waves 4-7 up rows
    const uint16_t* wsrc = (MODE == 0 && wave >= 4) ? a.w1 : a.w0;

    const TailSplit ts = tail_split(total, nblk, np > 3 ? np / 2 : 1, a.part_cap);
    const int ntasks = ts.nfull + ts.rtail * ts.S;

    // B-tile row of this lane's fragment ni (mode 0: gate rows, then the
    // matching up rows 128 further)
    auto brow = [&](int ni) __attribute__((always_inline)) {
        return (MODE == 0) ? ni * 128 + wi * 32 + (lane & 31) : wi * 64 + ni * 32 + (lane & 31);
    };

    // task t: whole tile, or part sp of tail tile j (K steps [kb, ke), kb
    // even); its tile and this lane's copy offsets.  Copy rows r_i = 32w + 8i
    // + lane/8 take logical chunk (lane%8) ^ ((r_i/2)&7): chunk kc0 for even
    // i, kc0 ^ 4 for odd i (byte offset kodd further).  Rows that follow one
    // another in memory (B rows; A rows of the down pass) keep the offset of
    // row r_0 and the count of rows left from it; gathered A rows (gate/up)
    // keep one offset per i.
    constexpr bool AG = MODE == 0;                // A rows gathered through perm
    int c_kb, c_ke, c_kend, c_pi, c_nt, c_p0, c_rows, c_e;
    uint32_t c_a[AG ? 4 : 1], c_b0;
    int c_an, c_bn;
    const int kc0 = (lane & 7) ^ ((lane >> 4) & 3);
    const int kodd = (((kc0 ^ 4) - kc0) * 16);
    // FAST copies: the per-lane part of a copy offset does not depend on the
    // task (row r0 of the tile and the lane's chunk; odd i take chunk ^ 4)
    const int r0c = wave * 32 + (lane >> 3);
    const uint32_t laneB_e = (uint32_t)((MODE == 0) ? (r0c & 127) : r0c) * row_bytes + (uint32_t)kc0 * 16u;
    const uint32_t laneB_o = laneB_e + (uint32_t)kodd;
    const uint32_t laneA_e = (uint32_t)r0c * row_bytes + (uint32_t)kc0 * 16u;
    const uint32_t laneA_o = laneA_e + (uint32_t)kodd;
    constexpr uint32_t TNB = (MODE == 0) ? 128u : (uint32_t)MF_BN;   // B-tile rows per N-tile step
    auto setup = [&](int t) __attribute__((always_inline)) {
        int L = t;
        c_kb = 0;
        c_ke = nk;
        c_pi = -1;
        if (t >= ts.nfull) {
            const int q = t - ts.nfull, j = q % ts.rtail, sp = q / ts.rtail;
            L = ts.nfull + j;
            c_kb = 2 * (int)((long)np * sp / ts.S);
            c_ke = min(nk, 2 * (int)((long)np * (sp + 1) / ts.S));
            c_pi = j * ts.S + sp;
        }
        c_kend = min(K, c_ke * MF_BK);           // element bound of the task's K range
        int mt;
        grouped_tile(L, n_mt, nN, mt, c_nt);
        c_e = a.tiles[mt];
        c_p0 = a.tiles[a.max_mt + mt];
        c_rows = a.tiles[2 * a.max_mt + mt];
        const int r0 = wave * 32 + (lane >> 3);
        if constexpr (AG) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 8 * i;
                const uint32_t cb = (uint32_t)(kc0 ^ ((i & 1) << 2)) * 16u;
                c_a[i] = r < c_rows ? (uint32_t)(a.perm[c_p0 + r] / a.topk) * row_bytes + cb : MF_OOB;
            }
        } else {
            c_a[0] = (uint32_t)(c_p0 + r0) * row_bytes + (uint32_t)kc0 * 16u;
        }
        c_an = c_rows - r0;
        const int n0 = (MODE == 0) ? c_nt * 128 + (r0 & 127) : c_nt * MF_BN + r0;
        c_b0 = (uint32_t)n0 * row_bytes + (uint32_t)kc0 * 16u;
        c_bn = N - n0;
    };

    if (slot >= ntasks) return;
    // With two or more K pairs per task (tail parts are cut to at least two)
    // the copy stream runs on from one task into the next: the last pairs'
    // steps issue the next task's A0, B0 and B1 into the slots the stream
    // reaches, so a new tile starts with its first pair already landed.  With
    // a single pair every task fills its slots from scratch.
    const bool stream = np >= 2;
    uint16_t* const sA0 = smem;
    uint16_t* const sB0 = smem + MF_AS * MF_PSLOT;
    int ca = 0, cb = 0, nb = 1, tb = 2;               // current A slot; current, next, third B slot
    setup(slot);
    bool first = true;
    for (int task = slot; task < ntasks; task += nblk) {
        const int kb = c_kb, ke = c_ke, kend = c_kend;
        uint32_t aoff[AG ? 4 : 1];
#pragma unroll
        for (int i = 0; i < (AG ? 4 : 1); ++i) aoff[i] = c_a[i];
        const uint32_t boff0 = c_b0;
        const int an = c_an, bn = c_bn;
        const int pi = c_pi, nt = c_nt, p0 = c_p0, rows = c_rows;
        const int32x4_t RB = make_desc(wsrc + (size_t)c_e * N * K, wmat);
        const int P = (ke - kb + 1) / 2;         // pairs of the task (an odd last step runs on zeros)
        const bool has_next = task + nblk < ntasks;
        // FAST: the tile's rows fill nf 32-row token fragments; group 0 takes
        // the first ceil(nf/2) of them, group 1 the rest (a full tile: 4 and
        // 4).  A group reads and multiplies only its own fragments, so the
        // padding of a ragged last tile costs at most one fragment instead of
        // up to 255 rows; the copies (and the barriers) stay the same for every
        // tile.  Other K keep four fragments per group (their variant would
        // not fit the register file with the smaller ones beside it).
        const int nf = (rows + 31) >> 5;
        const int mi0 = FAST ? (nf + 1) >> 1 : 4;
        const int my_mi = __builtin_amdgcn_readfirstlane(grp == 0 ? mi0 : (FAST ? nf - mi0 : 4));
        const int rbase = grp == 0 ? 0 : 32 * mi0;   // first tile row of this group
        floatx16 acc[4][2];
        bf16x8_t fa[2][4], fb[2][2];

        // this wave's 4 copies of pair j (K from element k0) of A (or B) of a
        // task with the given offsets, into the pair slot at `base`: rows
        // 32w + 8i .., the pair's 128-byte line of each
        auto copies = [&](bool isb, int k0, int kendv, const uint32_t* ao, uint32_t bo0, int anv, int bnv,
                          const int32x4_t& rb, uint16_t* base) __attribute__((always_inline)) {
            const uint32_t kbyte = (uint32_t)k0 * 2u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kok = k0 + 8 * (kc0 ^ ((i & 1) << 2)) < kendv;
                const uint32_t step = 8u * (uint32_t)i * row_bytes + ((i & 1) ? (uint32_t)kodd : 0u);
                uint32_t o;
                if (isb) o = 8 * i < bnv ? bo0 + step : MF_OOB;
                else if constexpr (AG) o = ao[i];
                else o = 8 * i < anv ? ao[0] + step : MF_OOB;
                dma16(isb ? rb : RA, (kok && o != MF_OOB) ? o + kbyte : MF_OOB,
                      lds_addr(&base[(wave * 32 + 8 * i) * MF_PK]));
            }
        };
        auto issue = [&](bool isb, int j, uint16_t* base) __attribute__((always_inline)) {
            copies(isb, (kb + 2 * j) * MF_BK, kend, aoff, boff0, an, bn, RB, base);
        };
        // pair j of the next task, from the offsets setup() left in c_*
        auto issue_next = [&](bool isb, int j, uint16_t* base) __attribute__((always_inline)) {
            const int32x4_t rbn = make_desc(wsrc + (size_t)c_e * N * K, wmat);
            copies(isb, (c_kb + 2 * j) * MF_BK, c_kend, c_a, c_b0, c_an, c_bn, rbn, base);
        };
        // fragments of one K step: half h (the first or second 32 of K) of the
        // pair slots sa (A) and sb (B), for the MI token fragments of this group
        auto read = [&](auto mic, const uint16_t* sa, const uint16_t* sb, int h) __attribute__((always_inline)) {
            constexpr int MI = decltype(mic)::value;
            if constexpr (MI > 0) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int ch = h * 4 + ks * 2 + (lane >> 5);
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        fa[ks][mi] = *reinterpret_cast<const bf16x8_t*>(&sa[swz2(rbase + mi * 32 + (lane & 31), ch)]);
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        fb[ks][ni] = *reinterpret_cast<const bf16x8_t*>(&sb[swz2(brow(ni), ch)]);
                }
            }
        };
        // transposed product: acc[mi][ni] is (B rows of fragment ni) x (tokens of fragment mi)
        // (FAST: copy i of the step goes out right after MFMA i * sp, i < 4:
        // sp = 1 at the first step of a pair, whose copies include group 0's
        // A(j+1) that must land within 1.5 phases, sp = 2 at the second; a
        // group with fewer fragments spaces them over the MFMAs it has, one
        // with none issues them back to back)
        auto mma = [&](auto mic, auto&& cp, auto sp) __attribute__((always_inline)) {
            constexpr int MI = decltype(mic)::value;
            constexpr int SP = decltype(sp)::value < (MI > 0 ? MI : 1) ? decltype(sp)::value : (MI > 0 ? MI : 1);
            if constexpr (MI == 0) {
                if constexpr (FAST) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        __builtin_amdgcn_sched_barrier(0);
                        cp(c);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                        for (int ni = 0; ni < 2; ++ni) {
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][ni], fa[ks][mi],
                                                                                   acc[mi][ni], 0, 0, 0);
                            const int idx = ks * 2 * MI + mi * 2 + ni;
                            if (FAST && idx % SP == 0 && idx / SP < 4) {
                                __builtin_amdgcn_sched_barrier(0);
                                cp(idx / SP);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
            }
        };

        // Copy schedule (groups of 4 copies per wave), one stream over the
        // pairs of the block's tasks: the first step of pair j issues A(j+1)
        // into the other A slot, the second step issues B(j+2) into the third
        // B slot; past the task's last pair these are the next task's A0, B0
        // and B1.  Both reuse slots whose last reads (step 2j - 1) both wave
        // groups have passed.  The barrier that ends group 0's memory phase of
        // step r is followed by group 1's reads of step r, the next one by
        // group 0's reads of step r + 1, so before it a wave must have landed
        // its copies of that step's pair.  The first step of a pair needs only
        // the pair itself (landed at the pair before); at the second step a
        // wave waits for A(j+1), the newest group the next pair needs: copies
        // complete in order, so until at most B(j+2) (if issued) is
        // outstanding.  In-order completion also makes that wait cover this
        // wave's epilogue stores of the previous tile; the barrier makes every
        // wave's copies visible and ends all LDS reads of the previous pair.
        //
        // FAST schedule (copies in the compute phases, 4 per wave per step):
        // at step 2j group 0 copies A(j+1) into the other A slot and group 1
        // B(j+2) into the third B slot; at step 2j+1 group 0 copies B(j+2) and
        // group 1 A(j+2) into this pair's A slot, which both groups have read
        // by then (group 1 runs one phase behind, so its compute phase of step
        // 2j+1 follows every read of pair j).  Group 0 waits at the end of
        // step 2j+1 until only B(j+2) is outstanding (A(j+1) landed); group 1
        // at the end of its memory phase of step 2j+1 until only B(j+2), its
        // newest, is outstanding (A(j+1), issued at step 2j-1, landed).  Past
        // the stream's end the copies are zero fills of slots nobody reads
        // again, so every step issues exactly four.
        if (first || !stream) {
            ca = 0; cb = 0; nb = 1; tb = 2;
            issue(false, 0, sA0);
            issue(true, 0, sB0);
            if (P > 1) issue(true, 1, sB0 + MF_PSLOT);
            if (FAST && grp == 1 && P > 1) issue(false, 1, sA0 + MF_PSLOT);
        }
        // the next task's loads go out behind this task's first copies and
        // land long before its own copies are issued
        if (has_next) setup(task + nblk);
        int32x4_t RBN = RB;                           // B descriptor of the next task
        if constexpr (FAST) RBN = make_desc(wsrc + (size_t)c_e * N * K, wmat);
        if (first || !stream) {
            wait_copies(P > 1 ? (FAST && grp == 1 ? 8 : 4) : 0);   // A0 and B0
            block_barrier();
            if (grp == 1) block_barrier();           // group 1 starts one phase later
        }
        first = false;
        // Per K step, each wave: memory phase (fragments of the step, then the
        // copies it issues), barrier, compute phase, barrier.
        auto step = [&](auto mic, int after1, int after2, auto&& cp, auto sp) __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): own fragments read
            if (after1 >= 0) wait_copies(after1);
            block_barrier();
            if (!FAST) __builtin_amdgcn_s_setprio(1);
            mma(mic, cp, sp);
            if (!FAST) __builtin_amdgcn_s_setprio(0);
            if (after2 >= 0) wait_copies(after2);
            block_barrier();
        };
        auto nocp = [](int) {};
        const bool nxt = stream && has_next;
        // FAST: offsets of this wave's four copies of A or B pair jb (this
        // task's, the next task's, or zero fills), its descriptor and LDS row
        uint32_t co[4];
        int32x4_t rd = RA;
        uint32_t lb = 0;
        auto prepA = [&](int jb, const uint16_t* slot) __attribute__((always_inline)) {
            const bool cur = jb < P;
            const int kp = cur ? kb + 2 * jb : c_kb + 2 * (jb - P);
            const bool on = cur || nxt;
            const uint32_t kbyte = (uint32_t)kp * (uint32_t)(MF_BK * 2);
            rd = RA;
            if constexpr (AG) {
                const uint32_t kadd = on ? kbyte : MF_OOB;
#pragma unroll
                for (int i = 0; i < 4; ++i) co[i] = (cur ? aoff[i] : c_a[i]) + kadd;
            } else {
                // rows past the group read the next rows of h (or zeros past its
                // end); their sums are never stored
                const uint32_t ub = on ? (uint32_t)(cur ? p0 : c_p0) * row_bytes + kbyte : MF_OOB;
#pragma unroll
                for (int i = 0; i < 4; ++i) co[i] = ((i & 1) ? laneA_o : laneA_e) + (ub + 8u * (uint32_t)i * row_bytes);
            }
            lb = lds_addr(&slot[(wave * 32) * MF_PK]);
        };
        auto prepB = [&](int jb, const uint16_t* slot) __attribute__((always_inline)) {
            const bool cur = jb < P;
            const int kp = cur ? kb + 2 * jb : c_kb + 2 * (jb - P);
            const bool on = cur || nxt;
            const uint32_t kbyte = (uint32_t)kp * (uint32_t)(MF_BK * 2);
            rd.x = cur ? RB.x : RBN.x;
            rd.y = cur ? RB.y : RBN.y;
            rd.z = cur ? RB.z : RBN.z;
            rd.w = RB.w;
            // rows past N are past the expert's range: zeros
            const uint32_t ub = on ? (uint32_t)(cur ? nt : c_nt) * TNB * row_bytes + kbyte : MF_OOB;
#pragma unroll
            for (int i = 0; i < 4; ++i) co[i] = ((i & 1) ? laneB_o : laneB_e) + (ub + 8u * (uint32_t)i * row_bytes);
            lb = lds_addr(&slot[(wave * 32) * MF_PK]);
        };
        auto cp = [&](int i) __attribute__((always_inline)) {
            dma16(rd, co[i], lb + (uint32_t)(i * 8 * MF_PK * 2));
        };
        // the K loop and the epilogue for a group of MI token fragments
        auto kloop = [&](auto mic) __attribute__((always_inline)) {
            constexpr int MI = decltype(mic)::value;
            if constexpr (MI > 0) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;
            }
            for (int j = 0; j < P; ++j) {
                const uint16_t* sa = sA0 + ca * MF_PSLOT;
                const uint16_t* sb = sB0 + cb * MF_PSLOT;
                if constexpr (FAST) {
                    read(mic, sa, sb, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (grp == 0) prepA(j + 1, sA0 + (ca ^ 1) * MF_PSLOT);
                    else prepB(j + 2, sB0 + tb * MF_PSLOT);
                    step(mic, -1, -1, cp, std::integral_constant<int, 1>{});
                    read(mic, sa, sb, 1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (grp == 0) prepB(j + 2, sB0 + tb * MF_PSLOT);
                    else prepA(j + 2, sA0 + ca * MF_PSLOT);
                    step(mic, grp == 0 ? -1 : 4, grp == 0 ? 4 : -1, cp, std::integral_constant<int, 2>{});
                } else {
                    read(mic, sa, sb, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (j + 1 < P) issue(false, j + 1, sA0 + (ca ^ 1) * MF_PSLOT);
                    else if (nxt) issue_next(false, 0, sA0 + (ca ^ 1) * MF_PSLOT);
                    step(mic, -1, -1, nocp, std::integral_constant<int, 1>{});
                    read(mic, sa, sb, 1);
                    __builtin_amdgcn_sched_barrier(0);
                    bool bnew = true;
                    if (j + 2 < P) issue(true, j + 2, sB0 + tb * MF_PSLOT);
                    else if (nxt) issue_next(true, j + 2 - P, sB0 + tb * MF_PSLOT);
                    else bnew = false;
                    // A(j+1) lands before the next pair; at the task's end without a
                    // streamed successor everything lands
                    const int after = (j + 1 < P || nxt) && bnew ? 4 : 0;
                    step(mic, grp == 0 ? -1 : after, after, nocp, std::integral_constant<int, 1>{});
                }
                ca ^= 1;
                const int t = cb;
                cb = nb;
                nb = tb;
                tb = t;
            }

            // ---- epilogue.  Accumulator element v of lane l: token row
            // rbase + mi*32 + l%32, B-tile row brow0(ni) + 8*(v/4) + 4*(l/32) + v%4,
            // i.e. four consecutive output columns per (v/4).
            const int c0 = 4 * (lane >> 5);
    #pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int row = rbase + mi * 32 + (lane & 31);
                if (pi >= 0) {
                    // a part of a split tail tile: raw fp32 sums, tile-local [row][B-tile row]
                    float* pt = a.part + (size_t)pi * (MF_BM * MF_BN) + row * MF_BN;
    #pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
    #pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int col = ((MODE == 0) ? ni * 128 + wi * 32 : wi * 64 + ni * 32) + 8 * q + c0;
                            *reinterpret_cast<float4*>(pt + col) = make_float4(
                                acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
                        }
                } else if (MODE == 0) {
                    // h = silu(g) * u, four bf16 (8 bytes) per lane and q
                    uint16_t* hrow = reinterpret_cast<uint16_t*>(a.out) + (size_t)(p0 + row) * N;
    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int f = nt * 128 + wi * 32 + 8 * q + c0;
                        float h[4];
    #pragma unroll
                        for (int j = 0; j < 4; ++j) h[j] = silu(acc[mi][0][4 * q + j]) * acc[mi][1][4 * q + j];
                        if (row < rows && f < N)
                            *reinterpret_cast<uint2*>(hrow + f) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                    }
                } else {
                    float* yrow = reinterpret_cast<float*>(a.out) + (size_t)(p0 + row) * N;
    #pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
    #pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = nt * MF_BN + wi * 64 + ni * 32 + 8 * q + c0;
                            if (row < rows && n < N)
                                *reinterpret_cast<float4*>(yrow + n) = make_float4(
                                    acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
                        }
                }
            }
        };
        if constexpr (FAST) {
            switch (my_mi) {
                case 4: kloop(std::integral_constant<int, 4>{}); break;
                case 3: kloop(std::integral_constant<int, 3>{}); break;
                case 2: kloop(std::integral_constant<int, 2>{}); break;
                case 1: kloop(std::integral_constant<int, 1>{}); break;
                default: kloop(std::integral_constant<int, 0>{}); break;
            }
        } else {
            kloop(std::integral_constant<int, 4>{});
        }
        // group 0 finished one phase earlier (its epilogue ran beside group 1's
        // last MFMAs); when the stream ends here its extra barrier pairs with
        // group 1's last one, as group 1 had the extra barrier at the start
        if (!nxt && grp == 0) block_barrier();
    }
    // the zero fills past the stream's end land before the block's LDS is released
    if constexpr (FAST) wait_copies(0);
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
    const int np = ((a.K + MF_BK - 1) / MF_BK + 1) / 2;      // K pairs, as the GEMM splits them
    const TailSplit ts = tail_split(n_mt * nN, G, np > 3 ? np / 2 : 1, a.part_cap);
    const int j = blockIdx.y;
    if (j >= ts.rtail) return;
    constexpr int NC = MODE == 0 ? 128 : MF_BN;      // output columns of a tile
    const int idx = (blockIdx.x * 256 + threadIdx.x) * 4;
    const int row = idx / NC, c = idx - row * NC;
    int mt, nt;
    grouped_tile(ts.nfull + j, n_mt, nN, mt, nt);
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
            if (f < N) reinterpret_cast<uint16_t*>(a.out)[orow + f] = (uint16_t)pack_bf16x2(silu(gv[i]) * uv[i], 0.f);
        } else {
            const int n = nt * MF_BN + c + i;
            if (n < N) reinterpret_cast<float*>(a.out)[orow + n] = gv[i];
        }
    }
}

// Small M-tiles (at most 64 rows: small expert groups and short remainders).
// Block tile 64 x 256 (gate/up: 128 gate + the 128 matching up rows), four
// waves side by side, each 64 x 64 = 2 x 2 accumulators of
// v_mfma_f32_32x32x16_bf16.  K is staged in pairs of steps like the 256-row
// kernel (128-byte LDS rows swizzled by (row/2)&7, every copy 8 rows x one
// whole line): two pair slots of A (8 KiB each) and of B (32 KiB each), 80 KiB
// of LDS so two blocks share a CU.  Such tiles stream each weight tile for
// few rows, so the kernel is bound by the weight stream, not the matrix cores.
//
// The copies go through registers, not buffer_load ... lds: each wave loads
// its ten lines of a K pair (2 of A, 8 of B; the weight lines non-temporal)
// into one of two register buffers, and writes them to the LDS pair slot just
// before the barrier that opens that pair.  A buffer is free again once
// written, so the loads of pair j+2 go out at the start of pair j and two
// pairs per wave are in flight through both K steps of a pair.  (The same
// tiles with LDS-direct copies and one pair in flight streamed the stack
// layer's weights ~11-14% slower; a third register buffer does not fit two
// blocks per CU.)  The loop body has no conditions: pairs past the last load
// as zeros (the range check) and multiply as zeros, so the compiler's wait
// counts see the same loads in flight at every step.
constexpr int MS_PSLOT_A = MS_BM * MF_PK;     // elements of an A pair slot
constexpr int MS_PSLOT_B = MF_BN * MF_PK;     // elements of a B pair slot
constexpr int MS_RING = 2;                    // register buffers (pairs)

template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_small_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][MS_PSLOT_A];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][MS_PSLOT_B];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, N = a.N;
    const int32_t* tl = a.tiles + 3 * a.max_mt + 1;
    const int max_st = a.max_st;
    const int n_st = tl[3 * max_st];
    const int nN = (MODE == 0) ? (N + 127) / 128 : (N + MF_BN - 1) / MF_BN;
    const int total = n_st * nN;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const int nk = (K + 31) / 32;
    const int P = (nk + 1) / 2;                   // K pairs (an odd last step runs on zeros)
    const __amdgpu_buffer_rsrc_t RA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.in), (short)0, (int)((uint32_t)a.in_rows * row_bytes), 0x00020000);
    const uint32_t wmat = (uint32_t)N * row_bytes;
    // copies: wave w fills A rows 16w + 8i + lane/8 (i = 0, 1) and B rows
    // 64w + 8i + lane/8 (i = 0..7), physical chunk lane%8 of the 128-byte row,
    // logical chunk kc0 for even i and kc0 ^ 4 for odd i (kodd bytes further)
    const int kc0 = (lane & 7) ^ ((lane >> 4) & 3);
    const int kodd = (((kc0 ^ 4) - kc0) * 16);
    const int crow = lane >> 3;

    for (int L = blockIdx.x; L < total; L += gridDim.x) {
        // small tiles of one expert next to each other: consecutive blocks
        // share the weight tile of one N column
        const int st_i = L % n_st, nt = L / n_st;
        const int e = tl[st_i];
        const int p0 = tl[max_st + st_i];
        const int rows = tl[2 * max_st + st_i];

        const uint16_t* wsrc = (MODE == 0 && wave >= 2) ? a.w1 : a.w0;
        const __amdgpu_buffer_rsrc_t RB = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(wsrc + (size_t)e * N * K), (short)0, (int)wmat, 0x00020000);
        uint32_t aoff[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = wave * 16 + 8 * i + crow;
            const uint32_t cb = (uint32_t)(kc0 ^ ((i & 1) << 2)) * 16u;
            if (r < rows) {
                const int src = (MODE == 0) ? a.perm[p0 + r] / a.topk : p0 + r;
                aoff[i] = (uint32_t)src * row_bytes + cb;
            } else {
                aoff[i] = MF_OOB;
            }
        }
        const int r0 = wave * 64 + crow;
        const int n0 = (MODE == 0) ? nt * 128 + (r0 & 127) : nt * MF_BN + r0;
        const uint32_t boff0 = (uint32_t)n0 * row_bytes + (uint32_t)kc0 * 16u;
        const int bn = N - n0;                    // B rows left from this lane's first
        floatx16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // this wave's ten lines of pair j into register buffer S
        u32x4_t ra[MS_RING][2], rb[MS_RING][8];
        auto load = [&](int j, auto slot) __attribute__((always_inline)) {
            constexpr int S = decltype(slot)::value;
            const int k0 = 2 * j * 32;
            const uint32_t kbyte = (uint32_t)k0 * 2u;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bool kok = k0 + 8 * (kc0 ^ ((i & 1) << 2)) < K;
                ra[S][i] = __builtin_amdgcn_raw_buffer_load_b128(
                    RA, (kok && aoff[i] != MF_OOB) ? aoff[i] + kbyte : MF_OOB, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool kok = k0 + 8 * (kc0 ^ ((i & 1) << 2)) < K;
                const uint32_t o = boff0 + 8u * (uint32_t)i * row_bytes + ((i & 1) ? (uint32_t)kodd : 0u);
                rb[S][i] = __builtin_amdgcn_raw_buffer_load_b128(RB, (kok && 8 * i < bn) ? o + kbyte : MF_OOB, 0,
                                                                 kNonTemporal);
            }
        };
        // register buffer S into LDS pair slot sl, each lane at the position
        // its line belongs to
        auto store = [&](auto slot, int sl) __attribute__((always_inline)) {
            constexpr int S = decltype(slot)::value;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                *reinterpret_cast<u32x4_t*>(&sA[sl][(wave * 16 + 8 * i) * MF_PK + 8 * lane]) = ra[S][i];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<u32x4_t*>(&sB[sl][(wave * 64 + 8 * i) * MF_PK + 8 * lane]) = rb[S][i];
        };
        auto brow = [&](int ni) {
            return (MODE == 0) ? ni * 128 + wave * 32 + (lane & 31) : wave * 64 + ni * 32 + (lane & 31);
        };
        // K step kt: per 16-K half, two token and two weight fragments, then
        // their four MFMAs
        auto step = [&](int kt) __attribute__((always_inline)) {
            const uint16_t* a_ = sA[(kt >> 1) & 1];
            const uint16_t* b_ = sB[(kt >> 1) & 1];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ch = (kt & 1) * 4 + ks * 2 + (lane >> 5);
                bf16x8_t fa[2], fb[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    fa[mi] = *reinterpret_cast<const bf16x8_t*>(&a_[swz2(mi * 32 + (lane & 31), ch)]);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    fb[ni] = *reinterpret_cast<const bf16x8_t*>(&b_[swz2(brow(ni), ch)]);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
            }
        };

        // the previous tile's fragment reads are done before slot 0 refills
        __syncthreads();
        static_for<0, MS_RING>([&](auto r) { load(decltype(r)::value, r); });
        store(ic<0>{}, 0);
        __syncthreads();
        // Pair j (in LDS slot j&1): load pair j+2 into the buffer pair j came
        // from (written to LDS in the previous iteration), the two K steps of
        // pair j, pair j+1 from its buffer into the other slot (whose pair j-1
        // every wave finished with before the previous barrier), barrier.
        const int Pp = (P + MS_RING - 1) / MS_RING * MS_RING;
        for (int j0 = 0; j0 < Pp; j0 += MS_RING) {
            static_for<0, MS_RING>([&](auto u) {
                constexpr int U = decltype(u)::value;
                const int j = j0 + U;
                load(j + MS_RING, u);
                __builtin_amdgcn_sched_barrier(0);   // the loads go out first
                step(2 * j);
                step(2 * j + 1);
                store(ic<(U + 1) % MS_RING>{}, (j + 1) & 1);
                __syncthreads();
            });
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

MfmaPlanArgs mfma_plan_args(int T, int k, int E, int tau, int tile_mode, int32_t* tiles, int max_mt) {
    return MfmaPlanArgs{tiles, tau, tile_mode, max_mt, mfma_max_small(T, k, E)};
}

hipError_t launch_mfma_plan(const int32_t* counts, const int32_t* offsets, int T, int k, int E, int tau,
                            int tile_mode, int32_t* tiles, int max_mt, hipStream_t s) {
    if (E > 256 || tile_mode < MFMA_TILES_BOTH || tile_mode > MFMA_TILES_BIG) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_plan_kernel, dim3(1), dim3(64), 0, s, counts, offsets, E,
                       mfma_plan_args(T, k, E, tau, tile_mode, tiles, max_mt));
    return hipGetLastError();
}

// T_tokens: the T of the layer (with k and E it sizes the small-tile list
// exactly as launch_mfma_plan did).
hipError_t launch_mfma_ffn(int mode, int tile_mode, const void* w0, const void* w1, const void* in, void* out,
                           const int32_t* perm, const int32_t* tiles, int N, int K, int topk, int T_tokens,
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
    a.max_st = mfma_max_small(T_tokens, topk, E);
    a.in_rows = in_rows;
    a.part = part;
    a.part_cap = part ? part_cap : 0;
    const int n_cu = cu_count();
    const int nN = mfma_ntiles_n(mode, N);
    hipError_t e = hipSuccess;
    if (tile_mode != MFMA_TILES_SMALL) {
        // big tiles: one 512-thread block per CU
        const int slots = max_mt * nN;
        const int grid = slots < n_cu ? slots : n_cu;
        // copies from the compute phase need whole K pairs and at least two of them
        const bool fast = K % (2 * MF_BK) == 0 && K >= 4 * MF_BK;
        if (mode == 0) {
            if (fast) hipLaunchKernelGGL((mfma_ffn_kernel<0, true>), dim3(grid), dim3(512), 0, s, a);
            else hipLaunchKernelGGL((mfma_ffn_kernel<0, false>), dim3(grid), dim3(512), 0, s, a);
        } else {
            if (fast) hipLaunchKernelGGL((mfma_ffn_kernel<1, true>), dim3(grid), dim3(512), 0, s, a);
            else hipLaunchKernelGGL((mfma_ffn_kernel<1, false>), dim3(grid), dim3(512), 0, s, a);
        }
        e = hipGetLastError();
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
    }
    if (tile_mode == MFMA_TILES_BIG) return e;
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
