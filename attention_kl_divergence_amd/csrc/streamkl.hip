// Fused attention-KL forward and backward for MI355X (gfx950, CDNA4), behind the
// C ABI declared in include/streamkl.h.
//
// Method: "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting
// Attention Distillation" (abstract) -- the KL between a teacher and a student
// attention row is reduced in one streaming pass over key tiles with online
// per-row state, and the backward recomputes both probability tiles from saved
// per-row log-normalisers instead of storing any N_Q x N_K intermediate.  The
// online normaliser is the running (max, sum) recurrence of "Online normalizer
// calculation for softmax" (listed among the works the StreamKL page builds on).
// The direction (teacher first) and nats follow "Lecture 05 - Where It All
// Lands", section 3.1.
//
// gfx950 mapping (all tiles are 32x32, wave64):
//  * Score tiles are produced transposed, C[y][x] = Y . X^T with
//    v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x2_f32 for fp32 inputs): the
//    "stationary" operand X (queries in the forward) sits in registers for the
//    whole kernel, the "streamed" operand Y (keys in the forward) is staged
//    through LDS, double-buffered, 16-byte coalesced loads.  In the accumulator
//    layout lane l owns column x = l % 32 and 16 rows y, so every lane keeps the
//    online state of ONE query over its own subset of keys with no cross-lane
//    traffic in the hot loop; the two half-waves are merged once at the end with
//    the associative merge of (max, normaliser, accumulators).
//  * The contraction index d is split so that half-wave h owns the contiguous
//    range [h*D/2, (h+1)*D/2): every operand load is a run of 16-byte vectors.
//  * Backward gradients G^T[d][x] += Y_s^T[d][y] . dS[y][x]: dS is used straight
//    from the accumulator registers as the B operand (the accumulator row
//    order is taken as the contraction order), and the matching transposed
//    student tile is read from the natural row-major LDS tile with
//    ds_read_b64_tr_b16, so no transposed copy is ever written.
//  * Workgroups are renumbered so that the blocks of one (batch, head) land on
//    the same XCD (the hardware deals workgroups round-robin over the 8 XCDs,
//    each with its own L2) and the heaviest blocks of every head are issued
//    first (block_order).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "streamkl.h"
#include "streamkl_internal.h"

namespace {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Stand-in score for a masked key: finite, so that 0 * score stays 0 and the
// running max of a lane that has seen no allowed key yet stays finite.
constexpr float kMasked = -1.0e30f;

#ifndef STREAMKL_WAVES
#define STREAMKL_WAVES 4
#endif
constexpr int kWaves = STREAMKL_WAVES;  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
// workgroups per CU the bf16 backward is built for: two waves per SIMD
constexpr int kBf16Blocks = 8 / kWaves;
// waves per SIMD the bf16 forward is built for (at most 168 registers each)
constexpr int kBf16FwdWaves = 3;
constexpr int kTile = 32;      // MFMA tile edge; each wave owns 32 stationary items
constexpr int kBlockX = kWaves * kTile;
constexpr int kBN = 32;        // streamed rows per pipeline stage
constexpr int kStateFloats = STREAMKL_STATE_FLOATS;  // (m_t, L, AT, AS, m_s, LS) per row
constexpr int kMaxSplit = 64;  // key splits of one split forward

// ---------------------------------------------------------------- type traits
template <typename T> struct Ty;
template <> struct Ty<bf16_t> {
    static constexpr int kBytes = 2;
    using Frag = bf16x8;
    __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // k-step ks of a half-wave span held as 16-byte vectors: 8 bf16 per step
    __device__ static inline Frag frag(const u32x4 *v, int ks) { return __builtin_bit_cast(Frag, v[ks]); }
    static constexpr int ksteps(int D) { return D / 16; }
};
template <> struct Ty<float> {
    static constexpr int kBytes = 4;
    using Frag = float;
    __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline Frag frag(const u32x4 *v, int ks) {
        // take the element as a scalar first: a bit_cast applied to a vector
        // element expression reads element 0 with this compiler
        const unsigned u = v[ks >> 2][ks & 3];
        return __builtin_bit_cast(float, u);
    }
    static constexpr int ksteps(int D) { return D / 2; }
};

// Barrier that publishes tiles filled by direct buffer->LDS loads.  Those loads
// count on the wave's vmcnt, and a workgroup barrier alone does not wait for
// them, so every wave first drains its own loads (vmcnt(0), lgkmcnt(0)); after
// the barrier every wave's share of the tiles is in LDS.
__device__ inline void dma_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    __syncthreads();
}

// 16-byte chunks in one half-wave span of a D-wide row
template <typename T, int D> constexpr int span_vecs() { return D * Ty<T>::kBytes / 32; }

// Work order of a launch with `per_head` blocks for each of `nheads` heads,
// ranked 0 (heaviest) .. per_head - 1 within a head.  The hardware deals
// workgroups round-robin over the 8 XCDs (block id b goes to XCD b % 8 as its
// (b / 8)-th block), each XCD with its own L2.  The heads are split over the
// XCDs so that all of a head's tiles go through one L2.  Head-major walks one
// head after the other, which keeps the blocks in flight on an XCD on as few
// heads as possible (their streamed tiles are shared in L2).  Rank-major walks
// the heaviest rank of every head of the XCD first; the host picks it when
// single blocks are long next to the whole launch, where head-major would
// start the heavy blocks of the last heads too late.
__device__ inline void block_order(int bid, int nblocks, int nheads, int per_head, bool rank_major, int &head,
                                   int &rank) {
    if ((nheads & 7) == 0) {
        const int hx = nheads >> 3, x = bid & 7, j = bid >> 3;
        if (rank_major) {
            rank = j / hx;
            head = x * hx + j % hx;
        } else {
            head = x * hx + j / per_head;
            rank = j % per_head;
        }
    } else if (rank_major) {
        rank = bid / nheads;
        head = bid % nheads;
    } else {
        const int x = bid & 7, j = bid >> 3, q = nblocks >> 3, r = nblocks & 7;
        const int wg = x * q + min(x, r) + j;  // contiguous block ranges per XCD
        head = wg / per_head;
        rank = wg % per_head;
    }
}

// Two waves share each SIMD.  With equal priorities the sequencer gives them
// issue slots in turn, and they tend to run the same phase (MFMAs, or the
// exponential arithmetic) at the same time.  Waves in odd hardware slots (bit 0
// of HW_ID.WAVE_ID) take a higher priority, so one wave of a pair runs ahead
// and the other fills the issue slots it leaves.  Used by the student-gradient
// backward only (1-2 % faster there); it slowed the teacher-gradient backward
// by about 5 % and the causal forward by about 1 %.
__device__ inline void stagger_priority() {
    if (__builtin_amdgcn_s_getreg(4 | (3 << 11)) & 1u) __builtin_amdgcn_s_setprio(2);  // hwreg(HW_ID, 0, 4)
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- LDS tiles
// A tile holds kBN rows of D elements back to back, without padding.  Each row
// is a run of 16-byte chunks and chunk c of row r sits at position c ^ swz(r).
// The swizzle keeps the two read patterns used on a tile free of bank conflicts
// on the 64-bank LDS: 16 lanes reading the same chunk of 16 consecutive rows
// (MFMA operand rows), and 16 lanes reading 32 contiguous bytes from each of 4
// consecutive rows (the transpose reads of the backward).  Tiles are filled by
// direct buffer->LDS loads, which place lane i's 16 bytes at slot base + 16 i,
// so each lane fetches the chunk of HBM that belongs at its slot.
template <typename T, int D>
struct Tile {
    static constexpr int kRowBytes = D * Ty<T>::kBytes;
    static constexpr int kChunks = kRowBytes / 16;  // 8, 16 or 32
    static constexpr int kBytes = kBN * kRowBytes;
    static_assert(kChunks == 8 || kChunks == 16 || kChunks == 32, "unsupported row width");
    __device__ static inline int swz(int r) {
        if constexpr (kChunks == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
        else return ((r & 3) << 2) | ((r >> 2) & 3);
    }
    __device__ static inline int chunk_off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }
};

// Rows [row0, row0 + kBN) of a [n, D] row-major matrix (row stride in elements)
// into an LDS tile, by direct buffer->LDS loads.  Rows past the end repeat the
// last row: they are always masked out before use, and finite values keep
// 0 * value = 0 in the contractions.
//
// The lane's part of every tile is fixed: DmaLanes holds, per load, the byte
// offset of the lane's chunk from the tile's first row, computed once per
// kernel.  Each tile then costs one wave-uniform buffer descriptor (scalar
// arithmetic) whose base is the tile's first row and whose size ends at its
// last valid row, so the hardware bounds every load to the tile.  The host
// keeps 32 row strides below 2^31 bytes, so the offsets fit in 32 bits.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

template <typename T, int D>
struct DmaLanes {
    using L = Tile<T, D>;
    static constexpr int kSlots = L::kBytes / 1024;  // 1 KiB per wave instruction
    static constexpr int kPerWave = (kSlots + kWaves - 1) / kWaves;
    uint32_t off[kPerWave];
    uint32_t sb;  // row stride in bytes
    __device__ inline DmaLanes(int64_t stride_n, int wv, int lane) {
        sb = (uint32_t)(stride_n * Ty<T>::kBytes);
#pragma unroll
        for (int k = 0; k < kPerWave; ++k) {
            const int pos = (k * kWaves + wv) * 64 + lane;  // chunk slot this lane fills
            const int r = pos / L::kChunks;
            const int c = (pos % L::kChunks) ^ L::swz(r);
            off[k] = (uint32_t)r * sb + (uint32_t)c * 16u;
        }
    }
};

template <typename T, int D>
__device__ inline void dma_tile(const DmaLanes<T, D> &ln, const T *base, int64_t stride_n, int row0, int nrows,
                                char *tile, int wv, int lane) {
    using L = Tile<T, D>;
    using DL = DmaLanes<T, D>;
    const int last = min(nrows - 1 - row0, kBN - 1);  // last row of the tile that exists (wave-uniform)
    if (last < 0) return;                              // no row (callers never ask for such a tile)
    const char *g0 = reinterpret_cast<const char *>(base + (int64_t)row0 * stride_n);
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(g0), (short)0,
                                                        (int)((uint32_t)last * ln.sb + L::kRowBytes), kBufferWord3);
#pragma unroll
    for (int k = 0; k < DL::kPerWave; ++k) {
        const int slot = k * kWaves + wv;  // wave-uniform
        if (DL::kSlots % kWaves != 0 && slot >= DL::kSlots) break;
        uint32_t o = ln.off[k];
        if (last < kBN - 1) {  // a tile crossing the end: rows past it read the last row
            const int r = (slot * 64 + lane) / L::kChunks;
            if (r > last) o -= (uint32_t)(r - last) * ln.sb;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(tile + slot * 1024),
                                                 16, o, 0, 0, 0);
    }
}

// The half-wave span [h*D/2, h*D/2 + D/2) of one global row into registers
// (zeros when the row does not exist).
template <typename T, int D>
__device__ inline void load_span_global(const T *row, int h, bool valid, u32x4 *out) {
    constexpr int NV = span_vecs<T, D>();
    const u32x4 *p = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(row) + h * (D / 2) * Ty<T>::kBytes);
    if (valid) {
#pragma unroll
        for (int v = 0; v < NV; ++v) out[v] = p[v];
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) out[v] = u32x4{0u, 0u, 0u, 0u};
    }
}

// The same span of row `row` of an LDS tile.
template <typename T, int D>
__device__ inline void load_span_lds(const char *tile, int row, int h, u32x4 *out) {
    constexpr int NV = span_vecs<T, D>();
#pragma unroll
    for (int v = 0; v < NV; ++v)
        out[v] = *reinterpret_cast<const u32x4 *>(tile + Tile<T, D>::chunk_off(row, h * NV + v));
}

// Row index (within a 32-row tile) of accumulator element i of half-wave h.
__device__ inline int acc_row(int i, int h) { return (i >> 2) * 8 + h * 4 + (i & 3); }

// ================================================================= forward
struct FwdParams {
    const void *q_t, *k_t, *q_s, *k_s;
    int64_t st[12];  // q_t(b,h,n), k_t(b,h,n), q_s(b,h,n), k_s(b,h,n), in elements
    int H, nheads, n_q, n_k, n_qblk;
    bool rank_major;
    float tau_t, tau_s;
    float *kl, *lse_t, *lse_s;
    // key range: split s of a block covers keys [k_begin + s k_chunk, that +
    // k_chunk) within [k_begin, k_end); k_begin and k_chunk are multiples of
    // the 32-key tile.  With state != null every (split, row) writes its raw
    // online state there ([n_split][rows][6]) instead of the finished row.
    int n_split, k_begin, k_end, k_chunk;
    float *state;
    // head mapping: KL head h reads head h / g of each tensor (q_t, k_t, q_s,
    // k_s); per-batch valid lengths (null: n_q, n_k)
    int g_qt, g_kt, g_qs, g_ks;
    const int *len_q, *len_k;
    // packed sequences: batch b's rows start at row cu[b] (null: padded)
    const int *cu_q, *cu_k;
};

// Valid length of batch b from a per-batch array (null: the full length),
// clamped to [0, n].
__device__ inline int batch_len(const int *len, int b, int n) {
    if (!len) return n;
    const int v = len[b];
    return v < 0 ? 0 : (v > n ? n : v);
}

// First row and valid length of batch b: packed sequences (cu = offsets
// [B + 1]) or padded ones (row 0, the length from `len` or n), clamped to n.
__device__ inline void batch_rows(const int *cu, const int *len, int b, int n, int &row0, int &nb) {
    if (cu) {
        row0 = cu[b];
        const int v = cu[b + 1] - row0;
        nb = v < 0 ? 0 : (v > n ? n : v);
    } else {
        row0 = 0;
        nb = batch_len(len, b, n);
    }
}


// C[y][x] = Y . X^T for one 32-row tile Y in LDS (pitch P) and this wave's
// stationary fragments X.
template <typename T, int D>
__device__ inline f32x16 tile_scores(const char *tile, const u32x4 *xv, int l32, int hf) {
    u32x4 yv[span_vecs<T, D>()];
    load_span_lds<T, D>(tile, l32, hf, yv);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < Ty<T>::ksteps(D); ++ks) acc = Ty<T>::mma(Ty<T>::frag(yv, ks), Ty<T>::frag(xv, ks), acc);
    return acc;
}

// Online state of one query over the keys one half-wave sees.  Scores are kept
// raw (x = q . k, unscaled); c = tau * log2(e) turns them into base-2 exponents.
// The sums are relative to reference maxima mt, ms: the result is exact for any
// reference that keeps the exponentials in range, so the reference is only
// moved when a tile would push a sum past 2^64 (see online_step).
struct Online {
    float mt, lt, at, as;  // teacher: reference max of x_t, sum e_t, sum e_t x_t, sum e_t x_s
    float ms, ls;          // student: reference max of x_s, sum e_s
    float nmt, nms;        // -c_t mt and -c_s ms, the exponent offsets of the references
};

// Exact update: the references become the running maxima and the sums are
// rescaled to them.  Masked keys are excluded.
template <bool MASK, bool CAUSAL>
__device__ inline void online_update(Online &o, f32x16 xt, f32x16 xs, float ct, float cs, int k0, int hf, int q,
                                     int n_k, int off) {
    unsigned okbits = 0xffffu;
    if (MASK) {
        okbits = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = k0 + acc_row(i, hf);
            const bool ok = key < n_k && (!CAUSAL || key <= q + off);
            okbits |= ok ? (1u << i) : 0u;
            xt[i] = ok ? xt[i] : kMasked;
            xs[i] = ok ? xs[i] : kMasked;
        }
    }
    float mxt = o.mt, mxs = o.ms;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        mxt = fmaxf(mxt, xt[i]);
        mxs = fmaxf(mxs, xs[i]);
    }
    const float rt = fast_exp2(ct * (o.mt - mxt));
    const float rs = fast_exp2(cs * (o.ms - mxs));
    o.mt = mxt;
    o.ms = mxs;
    const float nmt = -ct * mxt, nms = -cs * mxs;
    o.nmt = nmt;
    o.nms = nms;
    float lt = 0.f, ls = 0.f, at = 0.f, as = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float et = fast_exp2(fmaf(xt[i], ct, nmt));
        float es = fast_exp2(fmaf(xs[i], cs, nms));
        if (MASK && !((okbits >> i) & 1u)) {
            et = 0.f;
            es = 0.f;
        }
        lt += et;
        ls += es;
        at = fmaf(et, xt[i], at);
        as = fmaf(et, xs[i], as);
    }
    o.lt = fmaf(o.lt, rt, lt);
    o.at = fmaf(o.at, rt, at);
    o.as = fmaf(o.as, rt, as);
    o.ls = fmaf(o.ls, rs, ls);
}

// Steady-state update of an unmasked tile: exponentials against the current
// references, no maxima.  If any lane's tile sums are not safely below 2^64 (a
// score grew far past the reference, the references are still unset, or the
// row holds NaN), the whole wave redoes the tile with the exact update.
template <bool CAUSAL>
__device__ inline void online_step(Online &o, const f32x16 &xt, const f32x16 &xs, float ct, float cs, int k0, int hf,
                                   int q, int n_k, int off) {
    const float nmt = o.nmt, nms = o.nms;
    float lt = 0.f, ls = 0.f, at = 0.f, as = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float et = fast_exp2(fmaf(xt[i], ct, nmt));
        const float es = fast_exp2(fmaf(xs[i], cs, nms));
        lt += et;
        ls += es;
        at = fmaf(et, xt[i], at);
        as = fmaf(et, xs[i], as);
    }
    // Only the common branch below uses at and as, so the compiler would sink
    // their 32 FMAs past the branch, out of the block whose MFMAs they are
    // scheduled to hide under.  An empty statement that reads them keeps them
    // here (it emits no instruction).
    asm volatile("" ::"v"(at), "v"(as));
    const bool fine = (lt < 0x1p64f) && (ls < 0x1p64f);
    if (__builtin_amdgcn_ballot_w64(!fine) != 0) {
        online_update<false, CAUSAL>(o, xt, xs, ct, cs, k0, hf, q, n_k, off);
    } else {
        o.lt += lt;
        o.ls += ls;
        o.at += at;
        o.as += as;
    }
}

// One block = kWaves waves x 32 queries.  The key tiles stream through a two-stage
// LDS ring filled by direct buffer->LDS loads: a wave scores tile j and folds
// it into its running sums while the loads of tile j + 1 are in flight.  With
// one score tile live per wave (about 160 registers) three waves share each
// SIMD (bf16): while one waits for its MFMAs the others run exponentials.
// This beat a two-deep pipeline at two waves per SIMD (the MFMAs of tile j + 1
// interleaved with the sums of tile j), 4.84 -> 4.71 ms at 16384 x 16384.
template <typename T, int DT, int DS, bool CAUSAL>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? kBf16FwdWaves : 1) void streamkl_fwd_kernel(FwdParams p) {
    using TileT = Tile<T, DT>;
    using TileS = Tile<T, DS>;
    constexpr int STAGE = TileT::kBytes + TileS::kBytes;
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bh, rank;
    block_order(blockIdx.x, gridDim.x, p.nheads, p.n_qblk * p.n_split, p.rank_major, bh, rank);
    const int split = rank % p.n_split;
    const int qb = p.n_qblk - 1 - rank / p.n_split;  // high query blocks see the most keys under a causal mask
    const int hh = bh % p.H, bb = bh / p.H;
    const T *Qt = static_cast<const T *>(p.q_t) + bb * p.st[0] + (hh / p.g_qt) * p.st[1];
    const T *Kt = static_cast<const T *>(p.k_t) + bb * p.st[3] + (hh / p.g_kt) * p.st[4];
    const T *Qs = static_cast<const T *>(p.q_s) + bb * p.st[6] + (hh / p.g_qs) * p.st[7];
    const T *Ks = static_cast<const T *>(p.k_s) + bb * p.st[9] + (hh / p.g_ks) * p.st[10];
    const int64_t sqt = p.st[2], skt = p.st[5], sqs = p.st[8], sks = p.st[11];
    // valid rows of this batch (and, for packed sequences, where they start);
    // the per-row outputs keep the full n_q stride
    int rq0, rk0, n_q, n_k;
    batch_rows(p.cu_q, p.len_q, bb, p.n_q, rq0, n_q);
    batch_rows(p.cu_k, p.len_k, bb, p.n_k, rk0, n_k);
    const int off = n_k - n_q;
    Qt += (int64_t)rq0 * sqt;
    Qs += (int64_t)rq0 * sqs;
    Kt += (int64_t)rk0 * skt;
    Ks += (int64_t)rk0 * sks;

    const int q0w = qb * kBlockX + w * kTile;  // first query of this wave
    const int q = q0w + l32;                   // this lane's query
    const bool qv = q < n_q;
    const int qc = qv ? q : n_q - 1;
    const bool wave_live = q0w < n_q;
    const int qlast_w = min(n_q - 1, q0w + kTile - 1);

    const int qlast_wg = min(n_q - 1, qb * kBlockX + kBlockX - 1);
    // this block's keys: its split's range, cut at the causal end of its queries
    const int kb0 = p.k_begin + split * p.k_chunk;
    const int kend = min(min(p.k_end, kb0 + p.k_chunk), CAUSAL ? min(n_k, qlast_wg + off + 1) : n_k);
    const int ntile = kend > kb0 ? (kend - kb0 + kBN - 1) / kBN : 0;
    const int t0 = kb0 / kBN;  // tile t of the loop is global key tile t0 + t
    auto active = [&](int t) { return wave_live && (!CAUSAL || (t0 + t) * kBN <= qlast_w + off); };
    auto need_mask = [&](int t) {
        const int k0 = (t0 + t) * kBN;
        return (k0 + kBN > n_k) || (CAUSAL && k0 + kBN - 1 > q0w + off);
    };
    const DmaLanes<T, DT> lanes_t(skt, w, lane);
    const DmaLanes<T, DS> lanes_s(sks, w, lane);
    auto issue = [&](int t, char *stage) {
        dma_tile<T, DT>(lanes_t, Kt, skt, (t0 + t) * kBN, n_k, stage, w, lane);
        dma_tile<T, DS>(lanes_s, Ks, sks, (t0 + t) * kBN, n_k, stage + TileT::kBytes, w, lane);
    };

    if (ntile > 0) issue(0, smem);

    u32x4 qtv[span_vecs<T, DT>()], qsv[span_vecs<T, DS>()];
    load_span_global<T, DT>(Qt + (int64_t)qc * sqt, hf, qv, qtv);
    load_span_global<T, DS>(Qs + (int64_t)qc * sqs, hf, qv, qsv);

    const float ct = p.tau_t * kLog2e, cs = p.tau_s * kLog2e;
    Online o{kMasked, 0.f, 0.f, 0.f, kMasked, 0.f, -ct * kMasked, -cs * kMasked};

    dma_barrier();
    // one step per key tile.  Without a causal mask the loop runs two steps at
    // a time, so that the ring stage SL = it % 2 is a compile-time offset and
    // the LDS operand addresses need no per-tile arithmetic (measured slower
    // for the causal kernels, which keep one step per iteration).
    auto step = [&](int it, auto sl_tag) {
        constexpr int SL = decltype(sl_tag)::value;
        // the other stage was read in the previous step: load tile it + 1 there
        const int sl = SL >= 0 ? SL : (it & 1);
        if (it + 1 < ntile) issue(it + 1, smem + (sl ^ 1) * STAGE);
        const char *bc = smem + sl * STAGE;
        if (active(it)) {
            const int k0 = (t0 + it) * kBN;
            const f32x16 xt = tile_scores<T, DT>(bc, qtv, l32, hf);
            const f32x16 xs = tile_scores<T, DS>(bc + TileT::kBytes, qsv, l32, hf);
            if (need_mask(it)) online_update<true, CAUSAL>(o, xt, xs, ct, cs, k0, hf, q, n_k, off);
            else online_step<CAUSAL>(o, xt, xs, ct, cs, k0, hf, q, n_k, off);
        }
        dma_barrier();  // tile it + 1 is in LDS and every wave is done with tile it
    };
    if constexpr (CAUSAL) {
        for (int it = 0; it < ntile; ++it) step(it, std::integral_constant<int, -1>{});
    } else {
        int it = 0;
        for (; it + 1 < ntile; it += 2) {
            step(it, std::integral_constant<int, 0>{});
            step(it + 1, std::integral_constant<int, 1>{});
        }
        if (it < ntile) step(it, std::integral_constant<int, 0>{});
    }

    // merge the two half-waves (same query, disjoint key subsets)
    const float mt2 = __shfl_xor(o.mt, 32), lt2 = __shfl_xor(o.lt, 32);
    const float at2 = __shfl_xor(o.at, 32), as2 = __shfl_xor(o.as, 32);
    const float ms2 = __shfl_xor(o.ms, 32), ls2 = __shfl_xor(o.ls, 32);
    const float m = fmaxf(o.mt, mt2);
    const float w1 = fast_exp2(ct * (o.mt - m)), w2 = fast_exp2(ct * (mt2 - m));
    const float L = o.lt * w1 + lt2 * w2;
    const float AT = o.at * w1 + at2 * w2, AS = o.as * w1 + as2 * w2;
    const float mS = fmaxf(o.ms, ms2);
    const float v1 = fast_exp2(cs * (o.ms - mS)), v2 = fast_exp2(cs * (ms2 - mS));
    const float LS = o.ls * v1 + ls2 * v2;
    if (hf == 0 && q < p.n_q) {
        // rows past the batch's valid length, and rows with no allowed key,
        // are empty: KL 0, LSEs 0 (an empty state, L = 0, for partial states)
        const bool empty = !qv || L == 0.f;
        const int64_t row = ((int64_t)bb * p.H + hh) * p.n_q + q;
        if (p.state) {
            float *o6 = p.state + ((int64_t)split * p.nheads * p.n_q + row) * kStateFloats;  // [n_split][B H n_q][6]
            o6[0] = empty ? kMasked : m;
            o6[1] = empty ? 0.f : L;
            o6[2] = empty ? 0.f : AT;
            o6[3] = empty ? 0.f : AS;
            o6[4] = empty ? kMasked : mS;
            o6[5] = empty ? 0.f : LS;
        } else {
            const float lse_t = p.tau_t * m + logf(L);
            const float lse_s = p.tau_s * mS + logf(LS);
            // E_{P_t}[s_t - s_s] - LSE_t + LSE_s
            const float kl = (p.tau_t * AT - p.tau_s * AS) / L - lse_t + lse_s;
            p.kl[row] = empty ? 0.f : kl;
            p.lse_t[row] = empty ? 0.f : lse_t;
            p.lse_s[row] = empty ? 0.f : lse_s;
        }
    }
}

// Merge of partial online states.  Each of n_states states of a row holds, for
// its own key subset, reference maxima m_t, m_s of the raw scores and
//   L = sum 2^(c_t (x_t - m_t)),  AT = sum 2^(c_t (x_t - m_t)) x_t,
//   AS = sum 2^(c_t (x_t - m_t)) x_s,  LS = sum 2^(c_s (x_s - m_s))
// (c = tau log2 e).  Rescaled to the largest references they add up to the
// state of the union, which finishes into LSE_t, LSE_s and the row's KL.
__global__ __launch_bounds__(256) void streamkl_merge_kernel(const float *st, int n_states, int64_t rows,
                                                             float tau_t, float tau_s, float *kl_rows,
                                                             float *lse_t, float *lse_s) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    const float ct = tau_t * kLog2e, cs = tau_s * kLog2e;
    float m = kMasked, L = 0.f, AT = 0.f, AS = 0.f, mS = kMasked, LS = 0.f;
    for (int k = 0; k < n_states; ++k) {
        const float *o = st + ((int64_t)k * rows + row) * kStateFloats;
        const float m2 = o[0], L2 = o[1], AT2 = o[2], AS2 = o[3], mS2 = o[4], LS2 = o[5];
        const float mn = fmaxf(m, m2);
        const float w1 = fast_exp2(ct * (m - mn)), w2 = fast_exp2(ct * (m2 - mn));
        L = L * w1 + L2 * w2;
        AT = AT * w1 + AT2 * w2;
        AS = AS * w1 + AS2 * w2;
        m = mn;
        const float mSn = fmaxf(mS, mS2);
        LS = LS * fast_exp2(cs * (mS - mSn)) + LS2 * fast_exp2(cs * (mS2 - mSn));
        mS = mSn;
    }
    const float lt = tau_t * m + logf(L);
    const float ls = tau_s * mS + logf(LS);
    const bool empty = L == 0.f;  // no allowed key in any state: an empty row
    kl_rows[row] = empty ? 0.f : (tau_t * AT - tau_s * AS) / L - lt + ls;
    lse_t[row] = empty ? 0.f : lt;
    lse_s[row] = empty ? 0.f : ls;
}

// Deterministic sum of n fp32 values, one block: each thread accumulates a
// fixed, strided subset in fp64 with several loads in flight (16-byte loads
// when x is 16-byte aligned), then a fixed tree combines the partial sums.
__global__ __launch_bounds__(1024) void streamkl_sum_kernel(const float *x, int64_t n, float *out) {
    __shared__ double red[1024];
    double s = 0.0;
    int64_t i0 = 0;  // first element left to the scalar loop
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        constexpr int U = 8;
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
        const int64_t n4 = n / 4;
        int64_t j = threadIdx.x;
        for (; j + (U - 1) * 1024 < n4; j += U * 1024) {
            f32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = x4[j + u * 1024];
#pragma unroll
            for (int u = 0; u < U; ++u) s += ((double)v[u][0] + (double)v[u][1]) + ((double)v[u][2] + (double)v[u][3]);
        }
        for (; j < n4; j += 1024) {
            const f32x4 v = x4[j];
            s += ((double)v[0] + (double)v[1]) + ((double)v[2] + (double)v[3]);
        }
        i0 = n4 * 4;
    }
    constexpr int U = 8;
    int64_t i = i0 + threadIdx.x;
    for (; i + (U - 1) * 1024 < n; i += U * 1024) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = x[i + u * 1024];
#pragma unroll
        for (int u = 0; u < U; ++u) s += (double)v[u];
    }
    for (; i < n; i += 1024) s += (double)x[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int k = 512; k > 0; k >>= 1) {
        if ((int)threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = (float)red[0];
}

// ================================================================= backward
// One kernel body serves both gradients.  DKMODE = false: the stationary items
// x are queries and the streamed rows y are keys (output dq_s).  DKMODE = true:
// x are keys and y are queries (output dk_s).
struct BwdParams {
    const void *x_t, *x_s, *y_t, *y_s;
    int64_t st[12];  // x_t(b,h,n), x_s(b,h,n), y_t(b,h,n), y_s(b,h,n)
    int H, nheads, n_x, n_y, n_q, n_k, n_xblk;
    bool rank_major;
    float tau_t, tau_s;
    const float *lse_t, *lse_s, *g;
    const float *kl;  // per-row KL (first-argument gradients only)
    float g_scalar;
    void *out;
    // head mapping: KL head h reads head h / g of x_t, x_s, y_t, y_s; the
    // output has Hout heads, output head o sums KL heads [o group, (o + 1) group)
    int g_xt, g_xs, g_yt, g_ys, Hout, group;
    const int *len_q, *len_k;  // per-batch valid lengths (null: n_q, n_k)
    const int *cu_q, *cu_k;    // packed sequences: batch offsets [B + 1] (null: padded)
    // a group split over nsplit blocks of hsplit KL heads each, which write
    // fp32 partial gradients [nsplit][B Hout][n_x][DG] to `partial` (a later
    // launch sums them); n_xblk then counts n_x blocks times nsplit
    int nsplit, hsplit;
    float *partial;
};

// Range [ystart, yend) of streamed rows that stationary block xb meets: all of
// them, or under a causal mask (key j allowed for query i iff j <= i + n_k - n_q)
// the keys up to the block's last query (dq_s), the queries from the block's
// first key on, rounded down to a tile (dk_s).
template <bool CAUSAL, bool DKMODE>
__device__ inline void bwd_range(int n_q, int n_k, int n_y, int xb, int &ystart, int &yend) {
    const int off = n_k - n_q;
    ystart = 0;
    yend = n_y;
    if (CAUSAL) {
        if (!DKMODE) yend = min(n_k, min(n_q - 1, xb * kBlockX + kBlockX - 1) + off + 1);
        else ystart = (max(0, xb * kBlockX - off) / kBN) * kBN;
    }
}
// Streamed tiles of block xb at the full lengths (the work-order estimate).
template <bool CAUSAL, bool DKMODE>
__device__ inline int bwd_tiles(const BwdParams &p, int xb) {
    int ys, ye;
    bwd_range<CAUSAL, DKMODE>(p.n_q, p.n_k, p.n_y, xb, ys, ye);
    return (ye - ys + kBN - 1) / kBN;
}

// dS[y][x] = g * tau_s * (P_s - P_t) for one 32x32 tile, in fp32, with
// P = 2^(x * c - LSE * log2 e).  Per-query values (-LSE_t log2 e, -LSE_s log2 e,
// g tau_s) are per lane when the queries are the stationary items, else they
// come from the stage's LDS row-value block rv[3][kBN].
//
// FOLD: the upstream weight w = g tau_s is already inside the exponents as
// log2 |w| (both per-query values carry it), so dS / sign(w) = P'_s - P'_t and
// the sign is applied to the finished gradient; otherwise the third per-query
// value is w and multiplies the difference.
template <bool MASK, bool CAUSAL, bool DKMODE, int RS = kBN, bool FOLD = false>
__device__ inline void tile_ds(const f32x16 &xt, const f32x16 &xs, float ct, float cs, float nlt, float nls,
                               float gts, const float *rv, int y0, int hf, int x, int n_y, int off, float *dsv) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        f32x4 a_t, a_s, gg = f32x4{1.f, 1.f, 1.f, 1.f};
        if (DKMODE) {
            const int r0 = grp * 8 + hf * 4;
            a_t = *reinterpret_cast<const f32x4 *>(rv + r0);
            a_s = *reinterpret_cast<const f32x4 *>(rv + RS + r0);
            if (!FOLD) gg = *reinterpret_cast<const f32x4 *>(rv + 2 * RS + r0);
        } else {
            a_t = f32x4{nlt, nlt, nlt, nlt};
            a_s = f32x4{nls, nls, nls, nls};
            gg = f32x4{gts, gts, gts, gts};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = grp * 4 + e;
            const float pt = fast_exp2(fmaf(xt[i], ct, a_t[e]));
            const float ps = fast_exp2(fmaf(xs[i], cs, a_s[e]));
            float d = FOLD ? ps - pt : gg[e] * (ps - pt);
            if (MASK) {
                const int y = y0 + acc_row(i, hf);
                bool ok = y < n_y;
                if (CAUSAL) ok = ok && (DKMODE ? (x <= y + off) : (y <= x + off));
                d = ok ? d : 0.f;
            }
            dsv[i] = d;
        }
    }
}

// G^T[d][x] += Y_s^T[d][y] . dS[y][x].  dS is the B operand straight from the
// accumulator layout (its row order is the contraction order); the matching
// transposed student rows come from the row-major LDS tile via
// ds_read_b64_tr_b16 (fp32 inputs: one ds_read_b32 per k-step).
// First-argument (teacher) gradient of one 32x32 tile, in fp32:
//   dS_t[y][x] = w P_t (tau_t x_t - tau_s x_s - b),  b = LSE_t - LSE_s + KL
// with P_t = 2^(x_t c_t + a), a = -LSE_t log2 e (+ log2 |w| when FOLD, the sign
// of w then applied to the finished gradient).  Per-query values (a, -b, w)
// are per lane when the queries are the stationary items, else they come from
// the stage's LDS row-value block rv[3][RS].
template <bool MASK, bool CAUSAL, bool DKMODE, int RS, bool FOLD>
__device__ inline void tile_ds_first(const f32x16 &xt, const f32x16 &xs, float ct, float tau_t, float tau_s,
                                     float na, float nb, float wq, const float *rv, int y0, int hf, int x, int n_y,
                                     int off, float *dsv) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        f32x4 a_t, b_r, ww = f32x4{1.f, 1.f, 1.f, 1.f};
        if (DKMODE) {
            const int r0 = grp * 8 + hf * 4;
            a_t = *reinterpret_cast<const f32x4 *>(rv + r0);
            b_r = *reinterpret_cast<const f32x4 *>(rv + RS + r0);
            if (!FOLD) ww = *reinterpret_cast<const f32x4 *>(rv + 2 * RS + r0);
        } else {
            a_t = f32x4{na, na, na, na};
            b_r = f32x4{nb, nb, nb, nb};
            ww = f32x4{wq, wq, wq, wq};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = grp * 4 + e;
            const float pt = fast_exp2(fmaf(xt[i], ct, a_t[e]));
            const float l = fmaf(xs[i], -tau_s, fmaf(xt[i], tau_t, b_r[e]));
            float d = FOLD ? pt * l : ww[e] * pt * l;
            if (MASK) {
                const int y = y0 + acc_row(i, hf);
                bool ok = y < n_y;
                if (CAUSAL) ok = ok && (DKMODE ? (x <= y + off) : (y <= x + off));
                d = ok ? d : 0.f;
            }
            dsv[i] = d;
        }
    }
}

// Transposed student operands of one tile's gradient MFMAs (bf16): fragment
// [ks][t] holds Y_s^T rows t*32 + (lane % 32), contraction rows 16 ks + 8 (lane / 32)
// .. +8 of the tile, read from the row-major LDS tile with ds_read_b64_tr_b16.
template <int DS>
struct TrFrags {
    bf16x8 a[2][DS / kTile];
};
template <int DS>
__device__ inline void tr_load(TrFrags<DS> &f, const char *ys, int lane, int hf, int ks_lo, int ks_hi) {
    using L = Tile<bf16_t, DS>;
    const int trow = 4 * hf + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int ks = ks_lo; ks < ks_hi; ++ks) {
#pragma unroll
        for (int t = 0; t < DS / kTile; ++t) {
            const int r0 = 16 * ks + trow, col = t * kTile + tcol;
            const char *a0 = ys + L::chunk_off(r0, col >> 3) + (col & 7) * 2;
            const char *a1 = ys + L::chunk_off(r0 + 8, col >> 3) + (col & 7) * 2;
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(a0));
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(a1));
            const bf16x4 b0 = __builtin_bit_cast(bf16x4, v0), b1 = __builtin_bit_cast(bf16x4, v1);
            f.a[ks][t] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
    }
}

// G^T[d][x] += Y_s^T[d][y] . dS[y][x].  dS is the B operand straight from the
// accumulator layout (its row order is the contraction order); the matching
// transposed student rows come from the row-major LDS tile via
// ds_read_b64_tr_b16, loaded beforehand by tr_load (fp32 inputs: one
// ds_read_b32 per k-step, here).
template <typename T, int DS>
__device__ inline void tile_grad(f32x16 *G, const float *dsv, const void *trf, const char *ys, int hf, int l32) {
    using L = Tile<T, DS>;
    if constexpr (sizeof(T) == 2) {
        const TrFrags<DS> &f = *static_cast<const TrFrags<DS> *>(trf);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 bfrag;
#pragma unroll
            for (int e = 0; e < 8; ++e) bfrag[e] = (bf16_t)dsv[ks * 8 + e];
#pragma unroll
            for (int t = 0; t < DS / kTile; ++t) G[t] = Ty<bf16_t>::mma(f.a[ks][t], bfrag, G[t]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < DS / kTile; ++t) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = acc_row(i, hf), col = t * kTile + l32;
                const float a = *reinterpret_cast<const float *>(ys + L::chunk_off(r, col >> 2) + (col & 3) * 4);
                G[t] = Ty<float>::mma(a, dsv[i], G[t]);
            }
        }
    }
}

#ifndef STREAMKL_TR_EARLY
#define STREAMKL_TR_EARLY 0  // k-steps of transposed operands read before the dS arithmetic (0, 1 or 2; 0 measured best)
#endif
// The grouped-head kernels keep more state live across their head loop: with
// one k-step read early they spill less at the head boundaries.
constexpr int kTrEarlyGrouped = 1;
#ifndef STREAMKL_BWD_SUB
#define STREAMKL_BWD_SUB 2
#endif
// Streamed rows per pipeline stage of the backward: kBwdSub 32-row tiles
// share one barrier and one round of loads.
constexpr int kBwdSub = STREAMKL_BWD_SUB;
constexpr int kBwdRows = kBwdSub * kBN;

// One (stationary block, head) of the backward: the kBlockX stationary items
// x0 .. x0 + kBlockX - 1 (queries for dq_s, keys for dk_s) of head bh, with the
// other kind streamed through a two-stage LDS ring.  Two waves per SIMD overlap
// each other's MFMA and VALU phases.  GS: the upstream gradient is one scalar.
// FIRST: gradients with respect to the first (teacher) distribution, contracted
// with the teacher tiles (output width d_t) instead of the student ones.
template <typename T, int DT, int DS, bool CAUSAL, bool DKMODE, bool GS, bool FIRST, bool GRP>
__device__ __attribute__((always_inline)) inline void bwd_block(const BwdParams &p, int xb, int sp, int bh, char *smem,
                                                                float (*rowv)[3][kBwdRows]) {
    using TileT = Tile<T, DT>;
    using TileS = Tile<T, DS>;
    constexpr int PAIR = TileT::kBytes + TileS::kBytes;  // one 32-row tile of both tensors
    constexpr int STAGE = kBwdSub * PAIR;
    // fold w = g tau_s into the exponents whenever its sign is uniform over each
    // gradient row's contraction: always for query-major blocks (w belongs to
    // the stationary query), for key-major blocks when g is a scalar
    constexpr bool FOLD = !DKMODE || GS;
    constexpr int DG = FIRST ? DT : DS;  // width of the gradient rows
    constexpr int GOFF = FIRST ? 0 : TileT::kBytes;  // the contracted tile inside a PAIR

    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // output head `bh` (of B Hout): batch bb, head ho, fed by KL heads ho group + u
    const int ho = bh % p.Hout, bb = bh / p.Hout;
    const int64_t sxt = p.st[2], sxs = p.st[5], syt = p.st[8], sys = p.st[11];
    // valid lengths of this batch (the arrays keep the full n_q / n_x strides)
    // and, for packed sequences, the rows where they start
    int rq0, rk0, n_qb, n_kb;
    batch_rows(p.cu_q, p.len_q, bb, p.n_q, rq0, n_qb);
    batch_rows(p.cu_k, p.len_k, bb, p.n_k, rk0, n_kb);
    const int rx0 = DKMODE ? rk0 : rq0, ry0 = DKMODE ? rq0 : rk0;
    const bool packed_x = (DKMODE ? p.cu_k : p.cu_q) != nullptr;
    const int n_x = DKMODE ? n_kb : n_qb, n_y = DKMODE ? n_qb : n_kb, n_q = n_qb, off = n_kb - n_qb;
    const T *Xt, *Xs, *Yt, *Ys;  // the current KL head's tensors
    int64_t rowbase;              // per-query arrays of the current KL head
    auto set_head = [&](int hh) {
        Xt = static_cast<const T *>(p.x_t) + bb * p.st[0] + (hh / p.g_xt) * p.st[1] + (int64_t)rx0 * sxt;
        Xs = static_cast<const T *>(p.x_s) + bb * p.st[3] + (hh / p.g_xs) * p.st[4] + (int64_t)rx0 * sxs;
        Yt = static_cast<const T *>(p.y_t) + bb * p.st[6] + (hh / p.g_yt) * p.st[7] + (int64_t)ry0 * syt;
        Ys = static_cast<const T *>(p.y_s) + bb * p.st[9] + (hh / p.g_ys) * p.st[10] + (int64_t)ry0 * sys;
        rowbase = ((int64_t)bb * p.H + hh) * p.n_q;
    };

    const int x0w = xb * kBlockX + w * kTile;
    const int x = x0w + l32;
    const bool xv = x < n_x;
    const int xc = xv ? x : max(n_x - 1, 0);
    const bool wave_live = x0w < n_x;

    int ystart, yend;
    bwd_range<CAUSAL, DKMODE>(n_qb, n_kb, n_y, xb, ystart, yend);
    const int ntile = n_y > 0 ? max(0, (yend - ystart + kBN - 1) / kBN) : 0;
    auto active = [&](int t) {
        const int y0 = ystart + t * kBN;
        if (!wave_live) return false;
        if (!CAUSAL) return true;
        return DKMODE ? (y0 + kBN - 1 + off >= x0w) : (y0 <= min(n_q - 1, x0w + kTile - 1) + off);
    };
    auto need_mask = [&](int t) {
        const int y0 = ystart + t * kBN;
        bool m = y0 + kBN > n_y;
        if (CAUSAL) m = m || (DKMODE ? (x0w + kTile - 1 > y0 + off) : (y0 + kBN - 1 > x0w + off));
        return m;
    };
    const int nstage = (ntile + kBwdSub - 1) / kBwdSub;
    const DmaLanes<T, DT> lanes_t(syt, w, lane);
    const DmaLanes<T, DS> lanes_s(sys, w, lane);
    auto issue = [&](int st, int stage) {
#pragma unroll
        for (int sub = 0; sub < kBwdSub; ++sub) {
            const int t = st * kBwdSub + sub;
            if (t < ntile) {
                char *base = smem + stage * STAGE + sub * PAIR;
                dma_tile<T, DT>(lanes_t, Yt, syt, ystart + t * kBN, n_y, base, w, lane);
                dma_tile<T, DS>(lanes_s, Ys, sys, ystart + t * kBN, n_y, base + TileT::kBytes, w, lane);
            }
        }
    };
    // log2 |w| and sign(w) of the scalar upstream weight (folded key-major case)
    const float tau_g = FIRST ? p.tau_t : p.tau_s;  // the scale of the differentiated scores
    const float w_all = p.g_scalar * tau_g;
    const float lw_all = log2f(fabsf(w_all));
    // dk mode: the raw per-query values of query y0 + tid (tid < kBwdRows),
    // loaded before the stage's tile loads and turned into row values only
    // when they are stored, at the end of the stage: their wait then covers
    // them alone, not the tile loads issued after them
    float lt_r = 0.f, ls_r = 0.f, kl_r = 0.f, g_r = 0.f;
    bool y_ok = false;
    auto load_rows = [&](int st) {
        if (DKMODE && tid < kBwdRows) {
            const int y = ystart + st * kBwdRows + tid;
            y_ok = y < n_q;
            if (y_ok) {
                lt_r = p.lse_t[rowbase + y];
                ls_r = p.lse_s[rowbase + y];
                if (FIRST) kl_r = p.kl[rowbase + y];
                // per-row weight; the teacher kernels also take this path with a scalar g
                if (!FOLD) g_r = p.g ? p.g[rowbase + y] : p.g_scalar;
            }
        }
    };
    auto store_rows = [&](int stage) {
        if (DKMODE && tid < kBwdRows) {
            float rv0 = 0.f, rv1 = 0.f, rv2 = 0.f;
            if (y_ok) {
                rv0 = -lt_r * kLog2e;
                if (FIRST) rv1 = -(lt_r - ls_r + kl_r);
                else rv1 = -ls_r * kLog2e;
                if (FOLD) {
                    rv0 += lw_all;
                    if (!FIRST) rv1 += lw_all;
                } else {
                    rv2 = g_r * tau_g;
                }
            }
            rowv[stage][0][tid] = rv0;
            rowv[stage][1][tid] = rv1;
            if (!FOLD) rowv[stage][2][tid] = rv2;
        }
    };

    const float ct = p.tau_t * kLog2e, cs = p.tau_s * kLog2e;
    u32x4 xtv[span_vecs<T, DT>()], xsv[span_vecs<T, DS>()];
    float nlt = 0.f, nls = 0.f, gts = 0.f;  // per-lane row values (dq mode)
    float gsign = w_all < 0.f ? -1.f : 1.f;  // sign(w) applied to the finished gradient when folded
    f32x16 G[DG / kTile];
#pragma unroll
    for (int t = 0; t < DG / kTile; ++t) G[t] = f32x16{};

    // Start KL head hh: the first stage's loads, the stationary rows and the
    // per-lane row values.  G accumulates over the output head's KL heads;
    // when folded it holds the sum divided by the current head's sign, so a
    // change of sign between heads negates it.
    auto begin_head = [&](int hh, bool first_head) {
        set_head(hh);
        load_rows(0);
        issue(0, 0);
        load_span_global<T, DT>(Xt + (int64_t)xc * sxt, hf, xv, xtv);
        load_span_global<T, DS>(Xs + (int64_t)xc * sxs, hf, xv, xsv);
        if (!DKMODE && xv) {
            const float wq = ((GS || !p.g) ? p.g_scalar : p.g[rowbase + x]) * tau_g;
            const float lw = log2f(fabsf(wq));
            nlt = -p.lse_t[rowbase + x] * kLog2e + lw;
            if (FIRST) nls = -(p.lse_t[rowbase + x] - p.lse_s[rowbase + x] + p.kl[rowbase + x]);
            else nls = -p.lse_s[rowbase + x] * kLog2e + lw;
            const float sg = wq < 0.f ? -1.f : 1.f;
            if (!first_head && sg != gsign) {
#pragma unroll
                for (int t = 0; t < DG / kTile; ++t) G[t] = -G[t];
            }
            gsign = sg;
        }
        store_rows(0);
        dma_barrier();
    };

    auto ds_grad = [&](const f32x16 &cur_t, const f32x16 &cur_s, int it, int stage, int sub, bool m_cur,
                       auto early_tag) {
        constexpr int EARLY = decltype(early_tag)::value;  // k-steps of transposed reads before dS
        const int y0 = ystart + it * kBN;
        const float *rv = &rowv[DKMODE ? stage : 0][0][DKMODE ? sub * kBN : 0];
        const char *ys = smem + stage * STAGE + sub * PAIR + GOFF;
        // EARLY k-steps of the transposed operand reads can go out before the dS
        // arithmetic (which then hides their latency); the rest follow it
        TrFrags<(sizeof(T) == 2 ? DG : kTile)> trf;
        if constexpr (sizeof(T) == 2) {
            if (EARLY > 0) {
                tr_load<DG>(trf, ys, lane, hf, 0, EARLY);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        float dsv[16];
        if constexpr (FIRST) {
            if (m_cur)
                tile_ds_first<true, CAUSAL, DKMODE, kBwdRows, FOLD>(cur_t, cur_s, ct, p.tau_t, p.tau_s, nlt, nls,
                                                                    gts, rv, y0, hf, x, n_y, off, dsv);
            else
                tile_ds_first<false, CAUSAL, DKMODE, kBwdRows, FOLD>(cur_t, cur_s, ct, p.tau_t, p.tau_s, nlt, nls,
                                                                     gts, rv, y0, hf, x, n_y, off, dsv);
        } else {
            if (m_cur)
                tile_ds<true, CAUSAL, DKMODE, kBwdRows, FOLD>(cur_t, cur_s, ct, cs, nlt, nls, gts, rv, y0, hf, x, n_y,
                                                              off, dsv);
            else
                tile_ds<false, CAUSAL, DKMODE, kBwdRows, FOLD>(cur_t, cur_s, ct, cs, nlt, nls, gts, rv, y0, hf, x,
                                                               n_y, off, dsv);
        }
        if constexpr (sizeof(T) == 2) {
            if (EARLY < 2) tr_load<DG>(trf, ys, lane, hf, EARLY, 2);
        }
        tile_grad<T, DG>(G, dsv, &trf, ys, hf, l32);
    };

    // One ring stage: loads for the next stage, the tiles of this one, barrier.
    // PLAIN stages hold only tiles that are active and unmasked for this wave,
    // so their body has no branches (branches around the MFMA chain make the
    // compiler copy the gradient accumulators at every join).
    auto stage_body = [&](int st, auto plain_tag, int sc) {  // sc = st % 2, the ring slot
        constexpr bool PLAIN = decltype(plain_tag)::value;
        if (st + 1 < nstage) {
            load_rows(st + 1);
            issue(st + 1, sc ^ 1);
        }
#pragma unroll
        for (int sub = 0; sub < kBwdSub; ++sub) {
            const int it = st * kBwdSub + sub;
            const char *bc = smem + sc * STAGE + sub * PAIR;
            if (PLAIN) {
                const f32x16 cur_t = tile_scores<T, DT>(bc, xtv, l32, hf);
                const f32x16 cur_s = tile_scores<T, DS>(bc + TileT::kBytes, xsv, l32, hf);
                ds_grad(cur_t, cur_s, it, sc, sub, false,
                        std::integral_constant<int, GRP ? kTrEarlyGrouped : STREAMKL_TR_EARLY>{});
            } else if (it < ntile && active(it)) {
                const f32x16 cur_t = tile_scores<T, DT>(bc, xtv, l32, hf);
                const f32x16 cur_s = tile_scores<T, DS>(bc + TileT::kBytes, xsv, l32, hf);
                ds_grad(cur_t, cur_s, it, sc, sub, need_mask(it), std::integral_constant<int, 0>{});
            }
        }
        if (st + 1 < nstage) store_rows(sc ^ 1);
        dma_barrier();
    };
    // This wave's plain tiles are [t_lo, t_hi): tiles wholly inside the
    // streamed range and, under a causal mask, wholly on the allowed side.
    int t_lo = 0, t_hi = 0;
    if (wave_live) {
        t_hi = (n_y - ystart) / kBN;  // full tiles
        if (CAUSAL && !DKMODE) {
            // y0 + kBN - 1 <= x0w + off
            const int lim = x0w + off - (kBN - 1) - ystart;
            t_hi = min(t_hi, lim < 0 ? 0 : lim / kBN + 1);
        }
        if (CAUSAL && DKMODE) {
            // y0 >= x0w + kTile - 1 - off
            const int need = x0w + kTile - 1 - off - ystart;
            t_lo = need <= 0 ? 0 : (need + kBN - 1) / kBN;
        }
    }
    const int s_lo = min(nstage, (t_lo + kBwdSub - 1) / kBwdSub);
    const int s_hi = max(s_lo, min(nstage, t_hi / kBwdSub));
    // GRP: several KL heads feed this output head (a separate instantiation,
    // so that the single-head kernels keep their register allocation)
    const int ngroup = GRP ? p.group : 1;
    const int u0 = GRP ? sp * p.hsplit : 0, u1 = GRP ? min(ngroup, u0 + p.hsplit) : 1;
    for (int u = u0; u < u1; ++u) {
        begin_head(ho * ngroup + u, u == u0);
        for (int st = 0; st < s_lo; ++st) stage_body(st, std::false_type{}, st & 1);
        {
            // plain stages two at a time, so that the ring slot, and with it
            // every LDS address, is a compile-time offset
            int st = s_lo;
            if (st < s_hi && (st & 1)) stage_body(st++, std::true_type{}, 1);
            for (; st + 1 < s_hi; st += 2) {
                stage_body(st, std::true_type{}, 0);
                stage_body(st + 1, std::true_type{}, 1);
            }
            if (st < s_hi) stage_body(st, std::true_type{}, 0);
        }
        for (int st = s_hi; st < nstage; ++st) stage_body(st, std::false_type{}, st & 1);
    }

    if (FOLD) {
#pragma unroll
        for (int t = 0; t < DG / kTile; ++t) G[t] *= gsign;
    }
    if (!xv) {  // rows past the batch's valid length get zero gradients
#pragma unroll
        for (int t = 0; t < DG / kTile; ++t) G[t] = f32x16{};
    }
    if (GRP && p.partial && x < p.n_x) {
        // this split's share of the group: fp32 partial sums
        float *prow = p.partial + (((int64_t)sp * p.nheads + bh) * p.n_x + x) * DG;
#pragma unroll
        for (int t = 0; t < DG / kTile; ++t) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int d0 = t * kTile + grp * 8 + hf * 4;
                f32x4 o = {G[t][grp * 4 + 0], G[t][grp * 4 + 1], G[t][grp * 4 + 2], G[t][grp * 4 + 3]};
                *reinterpret_cast<f32x4 *>(prow + d0) = o;
            }
        }
    } else if (packed_x ? xv : x < p.n_x) {
        // padded outputs [B, Hout, n_x, DG] (rows past the valid length zeroed);
        // packed outputs [rows, Hout, DG], only this batch's valid rows
        T *orow = static_cast<T *>(p.out) + (packed_x ? ((int64_t)(rx0 + x) * p.Hout + ho) * DG
                                                      : (((int64_t)bb * p.Hout + ho) * p.n_x + x) * DG);
#pragma unroll
        for (int t = 0; t < DG / kTile; ++t) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int d0 = t * kTile + grp * 8 + hf * 4;
                if constexpr (sizeof(T) == 2) {
                    bf16x4 o = {(bf16_t)G[t][grp * 4 + 0], (bf16_t)G[t][grp * 4 + 1], (bf16_t)G[t][grp * 4 + 2],
                                (bf16_t)G[t][grp * 4 + 3]};
                    *reinterpret_cast<bf16x4 *>(orow + d0) = o;
                } else {
                    f32x4 o = {G[t][grp * 4 + 0], G[t][grp * 4 + 1], G[t][grp * 4 + 2], G[t][grp * 4 + 3]};
                    *reinterpret_cast<f32x4 *>(orow + d0) = o;
                }
            }
        }
    }
}

// One launch computes both gradients: each head has one work list holding its
// query blocks (dq_s) and its key blocks (dk_s), heaviest first (under a causal
// mask high query blocks see the most keys and low key blocks are seen by the
// most queries; for rectangular shapes the kind with the longer stream goes
// first), walked in the order of block_order.
template <typename T, int DT, int DS, bool CAUSAL, bool GS, bool FIRST, bool GRP>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? kBf16Blocks : 1) void streamkl_bwd_kernel(BwdParams pq,
                                                                                            BwdParams pk) {
    constexpr int STAGE = kBwdSub * (Tile<T, DT>::kBytes + Tile<T, DS>::kBytes);
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
    // per-query -LSE_t log2 e, -LSE_s log2 e, g tau_s of each stage's rows (dk_s blocks)
    __shared__ __attribute__((aligned(16))) float rowv[2][3][kBwdRows];
    if constexpr (!FIRST) stagger_priority();

    int bh, r;
    block_order(blockIdx.x, gridDim.x, pq.nheads, pq.n_xblk + pk.n_xblk, pq.rank_major, bh, r);
    // Rank r of a head's list: query blocks heaviest first (A, index i -> block
    // nq - 1 - i) merged with key blocks heaviest first (B, index j -> block j)
    // by streamed-tile count, ties alternating.  Both lists are non-increasing,
    // so the A count among the first r entries is found by bisection.
    const int nq = pq.n_xblk, nk = pk.n_xblk;
    auto wa = [&](int i) { return bwd_tiles<CAUSAL, false>(pq, nq - 1 - i); };
    auto wb = [&](int j) { return bwd_tiles<CAUSAL, true>(pk, j); };
    auto a_first = [&](int i, int j) {
        const int x = wa(i), y = wb(j);
        return x > y || (x == y && i <= j);
    };
    int lo = max(0, r - nk), hi = min(r, nq);
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a_first(mid, r - 1 - mid)) lo = mid + 1;
        else hi = mid;
    }
    const bool dk = !(r - lo >= nk || (lo < nq && a_first(lo, r - lo)));
    int idx = dk ? r - lo : nq - 1 - lo, sp = 0;
    if (GRP) {
        // split groups: consecutive work items are the splits of one block
        const int ns = dk ? pk.nsplit : pq.nsplit;
        sp = idx % ns;
        idx /= ns;
    }
    if (dk) bwd_block<T, DT, DS, CAUSAL, true, GS, FIRST, GRP>(pk, idx, sp, bh, smem, rowv);
    else bwd_block<T, DT, DS, CAUSAL, false, GS, FIRST, GRP>(pq, idx, sp, bh, smem, rowv);
}

// Sum of nsplit fp32 partial gradients [nsplit][n] into the output [n] in the
// input dtype, in a fixed order (n is a multiple of 4).
template <typename T>
__global__ __launch_bounds__(256) void streamkl_split_reduce_kernel(const float *partial, int nsplit, int64_t n,
                                                                    T *out) {
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
        f32x4 acc = *reinterpret_cast<const f32x4 *>(partial + i);
        for (int j = 1; j < nsplit; ++j) acc += *reinterpret_cast<const f32x4 *>(partial + (int64_t)j * n + i);
        if constexpr (sizeof(T) == 2) {
            bf16x4 o = {(bf16_t)acc[0], (bf16_t)acc[1], (bf16_t)acc[2], (bf16_t)acc[3]};
            *reinterpret_cast<bf16x4 *>(out + i) = o;
        } else {
            *reinterpret_cast<f32x4 *>(out + i) = acc;
        }
    }
}

}  // namespace

// Scratch of the allocation-free split forward: the split states live in
// this file-scope array (external linkage, so that the device code keeps it
// although no kernel names it).  Host code never passes `scratch` itself to a
// kernel (in host code the name is a stand-in, not a device address): the
// device address of each GPU's copy comes from hipGetSymbolAddress, looked up
// once per device with that device current, and is kept per device.
namespace streamkl_internal {
__device__ __align__(256) unsigned char scratch[STREAMKL_NOALLOC_SCRATCH_BYTES];
}

namespace {

// ================================================================= host side
struct Shape {
    int B, H, n_q, n_k, d_t, d_s;
};

// Head counts of q_t, k_t, q_s, k_s and the per-batch length arrays of a
// call (all H and null without a layout), checked.
struct Heads {
    int h[4];
    const int *len_q, *len_k;
    const int *cu_q, *cu_k;  // packed query / key sequences
    bool packed(int t) const { return (t % 2 == 0 ? cu_q : cu_k) != nullptr; }  // t: q_t, k_t, q_s, k_s
};
streamkl_status resolve_layout(const streamkl_layout *lay, int H, Heads &hd) {
    hd.len_q = hd.len_k = nullptr;
    hd.cu_q = hd.cu_k = nullptr;
    for (int t = 0; t < 4; ++t) hd.h[t] = H;
    if (!lay) return STREAMKL_OK;
    const int given[4] = {lay->heads_q_t, lay->heads_k_t, lay->heads_q_s, lay->heads_k_s};
    for (int t = 0; t < 4; ++t) {
        if (given[t] < 0) return STREAMKL_ERR_INVALID;
        hd.h[t] = given[t] ? given[t] : H;
    }
    // KL head h reads query head h / (H / Hq) and key head h / (H / Hk):
    // Hq divides H and Hk divides Hq in each model (grouped keys)
    for (int m = 0; m < 2; ++m) {
        const int hq = hd.h[2 * m], hk = hd.h[2 * m + 1];
        if (H % hq != 0 || hq % hk != 0) return STREAMKL_ERR_INVALID;
    }
    if (((uintptr_t)lay->seqlen_q) % 4 != 0 || ((uintptr_t)lay->seqlen_k) % 4 != 0) return STREAMKL_ERR_INVALID;
    if (((uintptr_t)lay->cu_seqlens_q) % 4 != 0 || ((uintptr_t)lay->cu_seqlens_k) % 4 != 0)
        return STREAMKL_ERR_INVALID;
    // a kind is either packed (offsets) or padded with lengths, not both
    if ((lay->cu_seqlens_q && lay->seqlen_q) || (lay->cu_seqlens_k && lay->seqlen_k)) return STREAMKL_ERR_INVALID;
    hd.len_q = lay->seqlen_q;
    hd.len_k = lay->seqlen_k;
    hd.cu_q = lay->cu_seqlens_q;
    hd.cu_k = lay->cu_seqlens_k;
    return STREAMKL_OK;
}

streamkl_status check_common(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                             streamkl_dtype dtype, const Shape &s, const int64_t *strides, float tau_t,
                             float tau_s, int causal, const Heads &hd, int64_t st[12]) {
    if (!q_t || !k_t || !q_s || !k_s) return STREAMKL_ERR_INVALID;
    if (dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) return STREAMKL_ERR_INVALID;
    if (s.B < 1 || s.H < 1 || s.n_q < 1 || s.n_k < 1 || s.d_t < 1 || s.d_s < 1) return STREAMKL_ERR_INVALID;
    if (!(tau_t >= 0.f) || !(tau_s >= 0.f) || !isfinite(tau_t) || !isfinite(tau_s)) return STREAMKL_ERR_INVALID;
    if (causal != 0 && causal != 1) return STREAMKL_ERR_INVALID;
    if (causal && s.n_q > s.n_k) return STREAMKL_ERR_INVALID;
    if (!streamkl_supported(dtype, s.d_t, s.d_s)) return STREAMKL_ERR_UNSUPPORTED;
    const int64_t elt = dtype == STREAMKL_BF16 ? 2 : 4;
    // grid size (a dispatch holds at most 2^32 - 1 work-items; the backward
    // grid has a block per query block and per key block of every head) and
    // 32-bit row arithmetic inside the kernels
    const int64_t nblk_q = ((int64_t)s.n_q + kBlockX - 1) / kBlockX, nblk_k = ((int64_t)s.n_k + kBlockX - 1) / kBlockX;
    if ((int64_t)s.B * s.H * (nblk_q + nblk_k) * kThreads > (int64_t)UINT32_MAX) return STREAMKL_ERR_INVALID;
    if ((int64_t)s.n_q + kBlockX > (int64_t)INT32_MAX / 2 || (int64_t)s.n_k + kBlockX > (int64_t)INT32_MAX / 2)
        return STREAMKL_ERR_INVALID;
    const int dims[4] = {s.d_t, s.d_t, s.d_s, s.d_s};
    const int ns[4] = {s.n_q, s.n_k, s.n_q, s.n_k};
    const void *ptrs[4] = {q_t, k_t, q_s, k_s};
    for (int t = 0; t < 4; ++t) {
        if (strides) {
            st[3 * t + 0] = strides[3 * t + 0];
            st[3 * t + 1] = strides[3 * t + 1];
            st[3 * t + 2] = strides[3 * t + 2];
            if (st[3 * t + 0] < 0 || st[3 * t + 1] < 0 || st[3 * t + 2] < dims[t]) return STREAMKL_ERR_INVALID;
        } else if (hd.packed(t)) {
            // packed sequences, contiguous [rows, heads, d]
            st[3 * t + 2] = (int64_t)hd.h[t] * dims[t];
            st[3 * t + 1] = dims[t];
            st[3 * t + 0] = 0;
        } else {
            st[3 * t + 2] = dims[t];
            st[3 * t + 1] = (int64_t)ns[t] * dims[t];
            st[3 * t + 0] = (int64_t)hd.h[t] * ns[t] * dims[t];
        }
        if (hd.packed(t)) st[3 * t + 0] = 0;  // rows are located by the offsets alone
        if (((uintptr_t)ptrs[t]) % 16 != 0) return STREAMKL_ERR_INVALID;
        // streamed tiles address 32 rows with 32-bit offsets
        if (st[3 * t + 2] * elt >= ((int64_t)1 << 26)) return STREAMKL_ERR_INVALID;
        for (int k = 0; k < 3; ++k)
            if ((st[3 * t + k] * elt) % 16 != 0) return STREAMKL_ERR_INVALID;
    }
    return STREAMKL_OK;
}

// Streamed tiles of each block (the same formulas as the kernels' ranges).
int64_t fwd_block_tiles(const Shape &s, int causal, int qb) {
    const int off = s.n_k - s.n_q;
    const int qlast = std::min(s.n_q - 1, qb * kBlockX + kBlockX - 1);
    const int kend = causal ? std::min(s.n_k, qlast + off + 1) : s.n_k;
    return (kend + kBN - 1) / kBN;
}
int64_t bwd_block_tiles(const Shape &s, int causal, bool dk, int xb) {
    const int off = s.n_k - s.n_q;
    int ys = 0, ye = dk ? s.n_q : s.n_k;
    if (causal) {
        if (!dk) ye = std::min(s.n_k, std::min(s.n_q - 1, xb * kBlockX + kBlockX - 1) + off + 1);
        else ys = (std::max(0, xb * kBlockX - off) / kBN) * kBN;
    }
    return (ye - ys + kBN - 1) / kBN;
}
// Rank-major order when block lengths differ and the longest block is more
// than a quarter of what one workgroup slot of an XCD runs over the whole
// launch (32 CUs x 2 workgroups).  Equal blocks balance in either order and
// keep the head-major order for its L2 reuse.
bool want_rank_major(int64_t min_tiles, int64_t max_tiles, int64_t head_tiles, int64_t nheads) {
    const int64_t heads_per_xcd = (nheads + 7) / 8;
    return 2 * max_tiles > 3 * min_tiles && 4 * max_tiles > heads_per_xcd * head_tiles / 64;
}

typedef void (*fwd_launch_t)(const FwdParams &, int grid, hipStream_t);
typedef void (*bwd_launch_t)(const BwdParams &, const BwdParams &, int grid, hipStream_t);

template <typename T, int DT, int DS, bool C>
void launch_fwd(const FwdParams &p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((streamkl_fwd_kernel<T, DT, DS, C>), dim3(grid), dim3(kThreads), 0, s, p);
}
template <typename T, int DT, int DS, bool C, bool GS, bool FIRST, bool GRP = false>
void launch_bwd(const BwdParams &pq, const BwdParams &pk, int grid, hipStream_t s) {
    hipLaunchKernelGGL((streamkl_bwd_kernel<T, DT, DS, C, GS, FIRST, GRP>), dim3(grid), dim3(kThreads), 0, s, pq,
                       pk);
}

template <typename T, int DT, int DS>
fwd_launch_t pick_fwd2(int causal) {
    return causal ? launch_fwd<T, DT, DS, true> : launch_fwd<T, DT, DS, false>;
}
template <typename T, int DT, int DS>
bwd_launch_t pick_bwd2(int causal, bool gs, bool first, bool grp) {
    // grouped output heads and first-argument gradients take the per-row-weight
    // form only (no scalar fold in key-major blocks), which halves their
    // instantiations
    if (grp) {
        if (first) return causal ? launch_bwd<T, DT, DS, true, false, true, true>
                                 : launch_bwd<T, DT, DS, false, false, true, true>;
        return causal ? launch_bwd<T, DT, DS, true, false, false, true>
                      : launch_bwd<T, DT, DS, false, false, false, true>;
    }
    if (first) return causal ? launch_bwd<T, DT, DS, true, false, true> : launch_bwd<T, DT, DS, false, false, true>;
    if (gs) return causal ? launch_bwd<T, DT, DS, true, true, false> : launch_bwd<T, DT, DS, false, true, false>;
    return causal ? launch_bwd<T, DT, DS, true, false, false> : launch_bwd<T, DT, DS, false, false, false>;
}
template <typename T>
fwd_launch_t pick_fwd1(int d_t, int d_s, int causal) {
    if (d_t == 64 && d_s == 64) return pick_fwd2<T, 64, 64>(causal);
    if (d_t == 64 && d_s == 128) return pick_fwd2<T, 64, 128>(causal);
    if (d_t == 128 && d_s == 64) return pick_fwd2<T, 128, 64>(causal);
    if (d_t == 128 && d_s == 128) return pick_fwd2<T, 128, 128>(causal);
    return nullptr;
}
template <typename T>
bwd_launch_t pick_bwd1(int d_t, int d_s, int causal, bool gs, bool first, bool grp) {
    if (d_t == 64 && d_s == 64) return pick_bwd2<T, 64, 64>(causal, gs, first, grp);
    if (d_t == 64 && d_s == 128) return pick_bwd2<T, 64, 128>(causal, gs, first, grp);
    if (d_t == 128 && d_s == 64) return pick_bwd2<T, 128, 64>(causal, gs, first, grp);
    if (d_t == 128 && d_s == 128) return pick_bwd2<T, 128, 128>(causal, gs, first, grp);
    return nullptr;
}

// The forward over keys [k_begin, k_end) in n_split equal chunks: finished
// rows (state == null, one chunk) or raw online states ([n_split][rows][6]).
streamkl_status fwd_common(const void *q_t, const void *k_t, const void *q_s, const void *k_s, streamkl_dtype dtype,
                           int B, int H, int n_q, int n_k, int d_t, int d_s, const int64_t *strides,
                           const streamkl_layout *lay, float tau_t, float tau_s, int causal, int k_begin, int k_end,
                           int n_split, float *state, float *kl_rows, float *lse_t, float *lse_s, float *kl_sum,
                           void *stream) {
    const Shape s{B, H, n_q, n_k, d_t, d_s};
    FwdParams p{};
    if (B < 1 || H < 1) return STREAMKL_ERR_INVALID;
    Heads hd;
    streamkl_status rc = resolve_layout(lay, H, hd);
    if (rc != STREAMKL_OK) return rc;
    rc = check_common(q_t, k_t, q_s, k_s, dtype, s, strides, tau_t, tau_s, causal, hd, p.st);
    if (rc != STREAMKL_OK) return rc;
    p.g_qt = H / hd.h[0]; p.g_kt = H / hd.h[1]; p.g_qs = H / hd.h[2]; p.g_ks = H / hd.h[3];
    p.len_q = hd.len_q; p.len_k = hd.len_k;
    p.cu_q = hd.cu_q; p.cu_k = hd.cu_k;
    p.q_t = q_t; p.k_t = k_t; p.q_s = q_s; p.k_s = k_s;
    p.H = H; p.nheads = B * H; p.n_q = n_q; p.n_k = n_k;
    p.n_qblk = (n_q + kBlockX - 1) / kBlockX;
    if ((int64_t)B * H * p.n_qblk * n_split * kThreads > (int64_t)UINT32_MAX) return STREAMKL_ERR_INVALID;
    {
        int64_t mn = INT64_MAX, mx = 0, tot = 0;
        for (int qb = 0; qb < p.n_qblk; ++qb) {
            const int64_t t = fwd_block_tiles(s, causal, qb);
            mn = std::min(mn, t);
            mx = std::max(mx, t);
            tot += t;
        }
        p.rank_major = want_rank_major(mn, mx, tot, p.nheads);
    }
    p.tau_t = tau_t; p.tau_s = tau_s;
    p.kl = kl_rows; p.lse_t = lse_t; p.lse_s = lse_s;
    p.n_split = n_split;
    p.k_begin = k_begin;
    p.k_end = k_end;
    const int per = (k_end - k_begin + n_split - 1) / n_split;
    p.k_chunk = ((per + kBN - 1) / kBN) * kBN;
    p.state = state;
    fwd_launch_t fn = dtype == STREAMKL_BF16 ? pick_fwd1<bf16_t>(d_t, d_s, causal) : pick_fwd1<float>(d_t, d_s, causal);
    if (!fn) return STREAMKL_ERR_UNSUPPORTED;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (streamkl_internal::log_enabled())
        fprintf(stderr,
                "[streamkl] fwd %s B=%d H=%d n_q=%d n_k=%d d_t=%d d_s=%d causal=%d: %d waves x %d query rows per "
                "block, %d-key tiles, %d waves per SIMD; grid %d x %d threads; keys [%d, %d) in %d split(s) of %d; "
                "%s order%s\n",
                dtype == STREAMKL_BF16 ? "bf16" : "f32", B, H, n_q, n_k, d_t, d_s, causal, kWaves, kTile, kBN,
                dtype == STREAMKL_BF16 ? kBf16FwdWaves : 1, B * H * p.n_qblk * n_split, kThreads, k_begin, k_end,
                n_split, p.k_chunk, p.rank_major ? "rank-major" : "head-major", state ? ", raw states" : "");
    fn(p, B * H * p.n_qblk * n_split, hs);
    if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
    if (kl_sum && !state) {
        hipLaunchKernelGGL(streamkl_sum_kernel, dim3(1), dim3(1024), 0, hs, (const float *)kl_rows,
                           (int64_t)B * H * n_q, kl_sum);
        if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
    }
    return STREAMKL_OK;
}

// Splits of a head group of `group` KL heads whose output kind has `blocks`
// blocks: enough to give the launch about 1024 work items, each split a run of
// hsplit KL heads (every split non-empty).
void group_split(int64_t blocks, int group, int &nsplit, int &hsplit) {
    nsplit = 1;
    hsplit = group;
    if (group <= 1 || blocks >= 1024) return;
    const int want = (int)std::min<int64_t>(group, (1024 + blocks - 1) / blocks);
    hsplit = (group + want - 1) / want;
    nsplit = (group + hsplit - 1) / hsplit;
}
size_t split_bytes(int nsplit, int64_t nheads_out, int n_x, int dg) {
    return (size_t)nsplit * nheads_out * n_x * dg * sizeof(float);
}

// Both backward entry points: gradients of sum_r g_r KL_r with respect to the
// student (first = false, outputs d_s wide) or the teacher (first = true,
// outputs d_t wide, needs the forward's per-row KL).  Without grouped heads
// one launch holds the query-major and key-major blocks of every head; when
// several KL heads feed one output head (grouped keys, or fewer query heads
// in the differentiated model), each output block loops over its KL heads and
// the two kinds go in two launches.
streamkl_status bwd_common(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                           streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                           const int64_t *strides, const streamkl_layout *lay, float tau_t, float tau_s, int causal,
                           const float *lse_t, const float *lse_s, const float *kl_rows, const float *grad_rows,
                           float grad_scalar, void *dq_out, void *dk_out, bool first, void *workspace,
                           size_t workspace_bytes, void *stream) {
    const Shape s{B, H, n_q, n_k, d_t, d_s};
    if (B < 1 || H < 1) return STREAMKL_ERR_INVALID;
    if (workspace && ((uintptr_t)workspace) % 16 != 0) return STREAMKL_ERR_INVALID;
    Heads hd;
    streamkl_status rc = resolve_layout(lay, H, hd);
    if (rc != STREAMKL_OK) return rc;
    int64_t st[12];
    rc = check_common(q_t, k_t, q_s, k_s, dtype, s, strides, tau_t, tau_s, causal, hd, st);
    if (rc != STREAMKL_OK) return rc;
    if (!lse_t || !lse_s || !dq_out || !dk_out || (first && !kl_rows)) return STREAMKL_ERR_INVALID;
    if (!isfinite(grad_scalar)) return STREAMKL_ERR_INVALID;
    if (((uintptr_t)dq_out) % 16 != 0 || ((uintptr_t)dk_out) % 16 != 0) return STREAMKL_ERR_INVALID;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool bf = dtype == STREAMKL_BF16;
    // tensor head counts in the order of BwdParams: teacher/student of the kind
    const int hq_t = hd.h[0], hk_t = hd.h[1], hq_s = hd.h[2], hk_s = hd.h[3];
    BwdParams pp[2];
    for (int pass = 0; pass < 2; ++pass) {
        const bool dk = pass == 1;
        BwdParams &p = pp[pass];
        p = BwdParams{};
        // stationary operand first, streamed second
        const int xi = dk ? 1 : 0, yi = dk ? 0 : 1;  // 0 = queries, 1 = keys (index into q_t/k_t stride groups)
        const void *tq[2] = {q_t, k_t}, *sq[2] = {q_s, k_s};
        p.x_t = tq[xi]; p.x_s = sq[xi]; p.y_t = tq[yi]; p.y_s = sq[yi];
        for (int k = 0; k < 3; ++k) {
            p.st[0 + k] = st[3 * xi + k];        // teacher of the stationary kind
            p.st[3 + k] = st[3 * (2 + xi) + k];  // student of the stationary kind
            p.st[6 + k] = st[3 * yi + k];
            p.st[9 + k] = st[3 * (2 + yi) + k];
        }
        const int ht[2] = {hq_t, hk_t}, hs2[2] = {hq_s, hk_s};
        p.g_xt = H / ht[xi]; p.g_xs = H / hs2[xi]; p.g_yt = H / ht[yi]; p.g_ys = H / hs2[yi];
        p.Hout = first ? ht[xi] : hs2[xi];
        p.group = H / p.Hout;
        p.len_q = hd.len_q; p.len_k = hd.len_k;
        p.cu_q = hd.cu_q; p.cu_k = hd.cu_k;
        p.H = H; p.nheads = B * p.Hout; p.n_q = n_q; p.n_k = n_k;
        p.n_x = dk ? n_k : n_q;
        p.n_y = dk ? n_q : n_k;
        p.n_xblk = (p.n_x + kBlockX - 1) / kBlockX;
        p.tau_t = tau_t; p.tau_s = tau_s;
        p.lse_t = lse_t; p.lse_s = lse_s; p.g = grad_rows; p.g_scalar = grad_scalar;
        p.kl = kl_rows;
        p.out = dk ? dk_out : dq_out;
        p.nsplit = 1;
        p.hsplit = p.group;
        p.partial = nullptr;
    }
    const bool gs = grad_rows == nullptr;
    const bool grp = pp[0].group > 1 || pp[1].group > 1;
    bwd_launch_t fn = bf ? pick_bwd1<bf16_t>(d_t, d_s, causal, gs, first, grp)
                         : pick_bwd1<float>(d_t, d_s, causal, gs, first, grp);
    if (!fn) return STREAMKL_ERR_UNSUPPORTED;
    // work order: head-major or rank-major (block tiles at the full lengths)
    auto order = [&](bool use_q, bool use_k, int64_t nheads) {
        int64_t mn = INT64_MAX, mx = 0, tot = 0;
        for (int pass = 0; pass < 2; ++pass) {
            if (!(pass == 0 ? use_q : use_k)) continue;
            for (int xb = 0; xb < pp[pass].n_xblk; ++xb) {
                const int64_t t = bwd_block_tiles(s, causal, pass == 1, xb) * pp[pass].group;
                mn = std::min(mn, t);
                mx = std::max(mx, t);
                tot += t;
            }
        }
        return want_rank_major(mn, mx, tot, nheads);
    };
    if (!grp) {
        pp[0].rank_major = pp[1].rank_major = order(true, true, (int64_t)B * H);
        if (streamkl_internal::log_enabled())
            fprintf(stderr,
                    "[streamkl] bwd%s %s B=%d H=%d n_q=%d n_k=%d d_t=%d d_s=%d causal=%d: %d waves x %d rows per block, "
                    "%d-row streamed tiles, %d per stage, %d waves per SIMD; grid %d x %d threads (%d query-major + "
                    "%d key-major blocks per head), %s order, %s upstream gradient\n",
                    first ? " (first argument)" : "", bf ? "bf16" : "f32", B, H, n_q, n_k, d_t, d_s, causal, kWaves,
                    kTile, kBN, kBwdSub, bf ? kBf16Blocks * kWaves / 4 : 1, B * H * (pp[0].n_xblk + pp[1].n_xblk),
                    kThreads, pp[0].n_xblk, pp[1].n_xblk, pp[0].rank_major ? "rank-major" : "head-major",
                    gs ? "scalar" : "per-row");
        fn(pp[0], pp[1], B * H * (pp[0].n_xblk + pp[1].n_xblk), hs);
        if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
        return STREAMKL_OK;
    }
    for (int pass = 0; pass < 2; ++pass) {
        BwdParams &cur = pp[pass];
        // long groups over few output blocks: split each group over several
        // blocks when the caller gave room for their partial sums
        const int dg = first ? d_t : d_s;
        int ns = 1, hs_ = cur.group;
        // (packed outputs are written by the blocks themselves, never split)
        if (!hd.packed(pass)) group_split(cur.nheads * cur.n_xblk, cur.group, ns, hs_);
        if (ns > 1 && split_bytes(ns, cur.nheads, cur.n_x, dg) <= workspace_bytes && workspace) {
            cur.nsplit = ns;
            cur.hsplit = hs_;
            cur.partial = static_cast<float *>(workspace);
            cur.n_xblk *= ns;
        }
        BwdParams none = pp[1 - pass];
        none.n_xblk = 0;
        none.nheads = cur.nheads;
        cur.rank_major = none.rank_major = order(pass == 0, pass == 1, cur.nheads);
        if (streamkl_internal::log_enabled())
            fprintf(stderr,
                    "[streamkl] bwd%s %s %s pass, grouped heads (%d KL heads per output head, %d split(s) of %d): "
                    "grid %d x %d threads, %s order\n",
                    first ? " (first argument)" : "", bf ? "bf16" : "f32", pass == 0 ? "query-major" : "key-major",
                    cur.group, cur.nsplit, cur.hsplit, cur.nheads * cur.n_xblk, kThreads,
                    cur.rank_major ? "rank-major" : "head-major");
        if (pass == 0) fn(cur, none, cur.nheads * cur.n_xblk, hs);
        else fn(none, cur, cur.nheads * cur.n_xblk, hs);
        if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
        if (cur.nsplit > 1) {
            const int64_t n = (int64_t)cur.nheads * cur.n_x * dg;
            const unsigned grid = (unsigned)std::min<int64_t>((n / 4 + 255) / 256, 4096);
            if (bf)
                hipLaunchKernelGGL(streamkl_split_reduce_kernel<bf16_t>, dim3(grid), dim3(256), 0, hs, cur.partial,
                                   cur.nsplit, n, static_cast<bf16_t *>(cur.out));
            else
                hipLaunchKernelGGL(streamkl_split_reduce_kernel<float>, dim3(grid), dim3(256), 0, hs, cur.partial,
                                   cur.nsplit, n, static_cast<float *>(cur.out));
            if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
        }
    }
    return STREAMKL_OK;
}

// Workspace bytes of a grouped backward (0 when no group is split).
size_t bwd_ex_workspace(int B, int H, int n_q, int n_k, int d_t, int d_s, const streamkl_layout *lay, bool first) {
    if (B < 1 || H < 1 || n_q < 1 || n_k < 1) return 0;
    Heads hd;
    if (resolve_layout(lay, H, hd) != STREAMKL_OK) return 0;
    size_t need = 0;
    for (int pass = 0; pass < 2; ++pass) {
        const bool dk = pass == 1;
        const int hout = first ? hd.h[dk ? 1 : 0] : hd.h[dk ? 3 : 2];
        const int group = H / hout, n_x = dk ? n_k : n_q;
        const int nblk = B * hout * ((n_x + kBlockX - 1) / kBlockX);
        int ns = 1, hsp = group;
        if (!hd.packed(pass)) group_split(nblk, group, ns, hsp);
        if (ns > 1) need = std::max(need, split_bytes(ns, B * hout, n_x, first ? d_t : d_s));
    }
    return need;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (null on failure).
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(streamkl_internal::scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int streamkl_supported(streamkl_dtype dtype, int d_t, int d_s) {
    if (dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) return 0;
    const bool dt_ok = d_t == 64 || d_t == 128, ds_ok = d_s == 64 || d_s == 128;
    return dt_ok && ds_ok ? 1 : 0;
}

const char *streamkl_status_string(streamkl_status status) {
    switch (status) {
        case STREAMKL_OK: return "ok";
        case STREAMKL_ERR_INVALID: return "invalid argument";
        case STREAMKL_ERR_UNSUPPORTED: return "unsupported head dimension / dtype combination";
        case STREAMKL_ERR_WORKSPACE: return "workspace too small";
        case STREAMKL_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

size_t streamkl_bwd_workspace_size(int B, int H, int n_q, int n_k, int d_t, int d_s, streamkl_dtype dtype,
                                   int causal) {
    (void)B; (void)H; (void)n_q; (void)n_k; (void)d_t; (void)d_s; (void)dtype; (void)causal;
    return 0;
}

streamkl_status streamkl_fwd(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                             streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                             const int64_t *strides, float tau_t, float tau_s, int causal, float *kl_rows,
                             float *lse_t, float *lse_s, float *kl_sum, void *stream) {
    if (!kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    return fwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s, causal,
                      0, n_k, 1, nullptr, kl_rows, lse_t, lse_s, kl_sum, stream);
}

int streamkl_fwd_split_count(int B, int H, int n_q, int n_k, int causal) {
    if (B < 1 || H < 1 || n_q < 1 || n_k < 1) return 1;
    // One round of the bf16 forward is 256 CUs x 3 workgroups.  A launch that
    // fills whole rounds, or about three, needs no split.  A smaller launch is
    // split over the keys until it holds about 2048 blocks, keeping at least
    // 16 key tiles per split; measured best at 2 x 16 heads of 4096 x 4096 and
    // 8 x 16 heads of 512 queries x 16384 keys.  Under a causal mask the splits
    // are uneven (early query blocks need few keys), so a causal launch is
    // split only when it does not fill one round.
    const int64_t base = (int64_t)B * H * ((n_q + kBlockX - 1) / kBlockX);
    const int64_t round = 256 * kBf16FwdWaves;
    if (base % round == 0) return 1;
    const int64_t want = causal ? round : 2048;
    if (base >= want) return 1;
    int64_t n = (want + base - 1) / base;
    n = std::min<int64_t>(n, std::max<int64_t>(1, n_k / (16 * kBN)));
    return (int)std::min<int64_t>(n, kMaxSplit);
}

size_t streamkl_fwd_split_workspace_size(int B, int H, int n_q, int n_split) {
    if (B < 1 || H < 1 || n_q < 1 || n_split < 1) return 0;
    return (size_t)n_split * B * H * n_q * kStateFloats * sizeof(float);
}

streamkl_status streamkl_fwd_split(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                   streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                   const int64_t *strides, float tau_t, float tau_s, int causal, int n_split,
                                   void *workspace, size_t workspace_bytes, float *kl_rows, float *lse_t,
                                   float *lse_s, float *kl_sum, void *stream) {
    if (!kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    if (n_split < 1 || n_split > kMaxSplit) return STREAMKL_ERR_INVALID;
    if (n_split == 1)
        return fwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s,
                          causal, 0, n_k, 1, nullptr, kl_rows, lse_t, lse_s, kl_sum, stream);
    if (B < 1 || H < 1 || n_q < 1) return STREAMKL_ERR_INVALID;
    if (!workspace || ((uintptr_t)workspace) % 16 != 0) return STREAMKL_ERR_INVALID;
    if (workspace_bytes < streamkl_fwd_split_workspace_size(B, H, n_q, n_split)) return STREAMKL_ERR_WORKSPACE;
    float *state = static_cast<float *>(workspace);
    streamkl_status rc = fwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s,
                                    causal, 0, n_k, n_split, state, nullptr, nullptr, nullptr, nullptr, stream);
    if (rc != STREAMKL_OK) return rc;
    return streamkl_fwd_merge(state, n_split, (int64_t)B * H * n_q, tau_t, tau_s, kl_rows, lse_t, lse_s, kl_sum,
                              stream);
}

streamkl_status streamkl_fwd_split_noalloc(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                           streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                           const int64_t *strides, float tau_t, float tau_s, int causal,
                                           int n_split, float *kl_rows, float *lse_t, float *lse_s, float *kl_sum,
                                           void *stream) {
    if (!kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    if (n_split < 1 || n_split > kMaxSplit) return STREAMKL_ERR_INVALID;
    if (B < 1 || H < 1 || n_q < 1) return STREAMKL_ERR_INVALID;
    if (n_split == 1)  // one key range: no states, nothing to hold
        return fwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s,
                          causal, 0, n_k, 1, nullptr, kl_rows, lse_t, lse_s, kl_sum, stream);
    {
        // the argument checks of the split forward, on the host, before any HIP call
        Heads hd;
        resolve_layout(nullptr, H, hd);
        int64_t st[12];
        const streamkl_status rc = check_common(q_t, k_t, q_s, k_s, dtype, Shape{B, H, n_q, n_k, d_t, d_s},
                                                strides, tau_t, tau_s, causal, hd, st);
        if (rc != STREAMKL_OK) return rc;
    }
    if (streamkl_fwd_split_workspace_size(B, H, n_q, n_split) > STREAMKL_NOALLOC_SCRATCH_BYTES)
        return STREAMKL_ERR_WORKSPACE;
    void *ws = scratch_on_current_device();
    if (!ws) return STREAMKL_ERR_HIP;
    // every (split, row) state is written by the partial launch before the
    // merge reads it, so the array needs no clearing between calls
    return streamkl_fwd_split(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, tau_t, tau_s, causal,
                              n_split, ws, STREAMKL_NOALLOC_SCRATCH_BYTES, kl_rows, lse_t, lse_s, kl_sum, stream);
}

streamkl_status streamkl_fwd_partial(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                     streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                     const int64_t *strides, float tau_t, float tau_s, int causal, int k_begin,
                                     int k_end, float *state, void *stream) {
    if (!state || ((uintptr_t)state) % 16 != 0) return STREAMKL_ERR_INVALID;
    if (k_begin < 0 || k_end > n_k || k_begin >= k_end) return STREAMKL_ERR_INVALID;
    if (k_begin % kBN != 0 || (k_end % kBN != 0 && k_end != n_k)) return STREAMKL_ERR_INVALID;
    return fwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s, causal,
                      k_begin, k_end, 1, state, nullptr, nullptr, nullptr, nullptr, stream);
}

streamkl_status streamkl_fwd_merge(const float *states, int n_states, int64_t rows, float tau_t, float tau_s,
                                   float *kl_rows, float *lse_t, float *lse_s, float *kl_sum, void *stream) {
    if (!states || !kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    if (n_states < 1 || rows < 1 || (rows + 255) / 256 > (int64_t)INT32_MAX) return STREAMKL_ERR_INVALID;
    if (!(tau_t >= 0.f) || !(tau_s >= 0.f) || !isfinite(tau_t) || !isfinite(tau_s)) return STREAMKL_ERR_INVALID;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(streamkl_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, hs, states,
                       n_states, rows, tau_t, tau_s, kl_rows, lse_t, lse_s);
    if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
    if (kl_sum) {
        hipLaunchKernelGGL(streamkl_sum_kernel, dim3(1), dim3(1024), 0, hs, (const float *)kl_rows, rows, kl_sum);
        if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
    }
    return STREAMKL_OK;
}

streamkl_status streamkl_bwd(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                             streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                             const int64_t *strides, float tau_t, float tau_s, int causal, const float *lse_t,
                             const float *lse_s, const float *grad_rows, float grad_scalar, void *dq_s,
                             void *dk_s, void *stream) {
    return bwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s, causal,
                      lse_t, lse_s, nullptr, grad_rows, grad_scalar, dq_s, dk_s, false, nullptr, 0, stream);
}

streamkl_status streamkl_bwd_teacher(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                     streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                     const int64_t *strides, float tau_t, float tau_s, int causal,
                                     const float *lse_t, const float *lse_s, const float *kl_rows,
                                     const float *grad_rows, float grad_scalar, void *dq_t, void *dk_t,
                                     void *stream) {
    return bwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, nullptr, tau_t, tau_s, causal,
                      lse_t, lse_s, kl_rows, grad_rows, grad_scalar, dq_t, dk_t, true, nullptr, 0, stream);
}

streamkl_status streamkl_fwd_ex(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                const int64_t *strides, const streamkl_layout *layout, float tau_t, float tau_s,
                                int causal, float *kl_rows, float *lse_t, float *lse_s, float *kl_sum,
                                void *stream) {
    if (!kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    return fwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, layout, tau_t, tau_s, causal, 0,
                      n_k, 1, nullptr, kl_rows, lse_t, lse_s, kl_sum, stream);
}

size_t streamkl_bwd_ex_workspace_size(int B, int H, int n_q, int n_k, int d_t, int d_s,
                                      const streamkl_layout *layout, int first) {
    return bwd_ex_workspace(B, H, n_q, n_k, d_t, d_s, layout, first != 0);
}

streamkl_status streamkl_bwd_ex(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                const int64_t *strides, const streamkl_layout *layout, float tau_t, float tau_s,
                                int causal, const float *lse_t, const float *lse_s, const float *grad_rows,
                                float grad_scalar, void *dq_s, void *dk_s, void *workspace, size_t workspace_bytes,
                                void *stream) {
    return bwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, layout, tau_t, tau_s, causal,
                      lse_t, lse_s, nullptr, grad_rows, grad_scalar, dq_s, dk_s, false, workspace, workspace_bytes,
                      stream);
}

streamkl_status streamkl_bwd_teacher_ex(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                        streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                        const int64_t *strides, const streamkl_layout *layout, float tau_t,
                                        float tau_s, int causal, const float *lse_t, const float *lse_s,
                                        const float *kl_rows, const float *grad_rows, float grad_scalar, void *dq_t,
                                        void *dk_t, void *workspace, size_t workspace_bytes, void *stream) {
    return bwd_common(q_t, k_t, q_s, k_s, dtype, B, H, n_q, n_k, d_t, d_s, strides, layout, tau_t, tau_s, causal,
                      lse_t, lse_s, kl_rows, grad_rows, grad_scalar, dq_t, dk_t, true, workspace, workspace_bytes,
                      stream);
}

}  // extern "C"

namespace streamkl_internal {
bool log_enabled() {
    static const bool on = [] {
        const char *v = getenv("STREAMKL_LOG");
        return v != nullptr && *v != '\0' && strcmp(v, "0") != 0;
    }();
    return on;
}

hipError_t launch_row_sum(const float *x, int64_t n, float *out, hipStream_t s) {
    hipLaunchKernelGGL(streamkl_sum_kernel, dim3(1), dim3(1024), 0, s, x, n, out);
    return hipGetLastError();
}
}  // namespace streamkl_internal
