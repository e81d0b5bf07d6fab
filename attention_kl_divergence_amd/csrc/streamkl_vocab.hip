// Fused vocabulary-logit KL at temperature for MI355X (gfx950), behind the C
// ABI declared in include/streamkl.h (streamkl_vocab_*).
//
// Method: the distillation loss of "Lecture 05 - Where It All Lands", section
// 3.1 -- forward KL, teacher first, between the two output distributions over
// the vocabulary, both softened by dividing the logits by a temperature T --
// computed per row of a [rows, V] pair of logit matrices in one streaming pass
// with the online (reference max, normaliser) state of "Online normalizer
// calculation for softmax" (among the works the StreamKL page builds on), the
// same associative state the attention kernels keep per query row.  The T^2
// factor of section 3.3 belongs to the caller (through the upstream gradient).
//
// This is a bandwidth-bound workload (a few VALU operations and two exp2 per
// logit pair, no contraction), so it is built around HBM streaming, not MFMA:
//  * a row is owned by one wave (short rows) or one 4-wave workgroup (long
//    rows); each lane takes 8 consecutive logits of each operand per step as
//    16-byte loads (bf16; two for fp32), and a wave's step covers a contiguous
//    1 KiB (bf16) run of the row, several steps in flight per lane;
//  * every lane keeps its own state over its subset of the row, so the hot
//    loop has no cross-lane traffic; lanes and waves are merged once per row;
//  * the reference maxima are lazy: a lane re-bases only when a step's terms
//    sum past 2^64 (some logit far above the reference; also a lane's first
//    step), which is exact (terms up to 2^64 times the reference stay far
//    inside fp32) and needs no per-step maximum on the common path;
//  * the backward recomputes p and q from the saved log-normalisers and writes
//    dz_s (and dz_t) with 16-byte stores; no workspace, no atomics.
// Rows that are not 16-byte aligned (V or the leading dimension not a multiple
// of 8, or a misaligned base) stream their aligned body the same way when the
// rows of all operands start equally far from a 16-byte boundary (as two
// contiguous [rows, V] matrices do), with a few scalar logits before and
// after it; otherwise they take an element path, still coalesced across the
// wave.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "streamkl.h"
#include "streamkl_internal.h"

namespace {

typedef __bf16 bf16_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNoRef = -1.0e30f;  // reference of a lane that has seen no logit
constexpr float kPad = -2.0e30f;    // stand-in logit past the end of a row (generic path)
constexpr int kStep = 8;            // logits per lane per step
// steps in flight per lane: forward passes; gradient passes (16 bf16 or, at
// the same bytes in flight, 8 fp32 vectors)
constexpr int kUnrollState = 4;
template <typename T> constexpr int unroll_grad() { return sizeof(T) == 2 ? 8 : 4; }
// Waves per row: 1 (four short rows per 256-thread workgroup), or 4, 8, 16
// (one row per workgroup of 64 WPR threads).
template <int WPR> constexpr int block_threads() { return WPR >= 4 ? 64 * WPR : 256; }
template <int WPR> constexpr int rows_per_block() { return block_threads<WPR>() / (64 * WPR); }

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- 8-logit I/O
template <typename T> struct VIo;
// NT: a non-temporal access (the logits of a row are read once per pass and
// the gradients written once: streaming them past the caches leaves the
// caches to the rest of the traffic).  The fused launch's first pass keeps
// ordinary loads, so that its second pass finds the row in the caches.
template <> struct VIo<bf16_t> {
    struct Raw { u32x4 v; };
    template <bool NT = false>
    __device__ static inline Raw load(const bf16_t *p) {
        if constexpr (NT) return Raw{__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p))};
        else return Raw{*reinterpret_cast<const u32x4 *>(p)};
    }
    __device__ static inline void widen(const Raw &r, float z[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // the element is taken as a scalar before any bit cast (a bit cast
            // of a vector element expression can read element 0)
            const unsigned u = r.v[k];
            z[2 * k] = __builtin_bit_cast(float, u << 16);
            z[2 * k + 1] = __builtin_bit_cast(float, u & 0xffff0000u);
        }
    }
    template <bool NT = false>
    __device__ static inline void store(bf16_t *p, const float z[8]) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bf16_t lo = (bf16_t)z[2 * k], hi = (bf16_t)z[2 * k + 1];
            o[k] = (unsigned)__builtin_bit_cast(unsigned short, lo) |
                   ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
        }
        if constexpr (NT) __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(p));
        else *reinterpret_cast<u32x4 *>(p) = o;
    }
    __device__ static inline float load1(const bf16_t *p) { return (float)*p; }
    __device__ static inline void store1(bf16_t *p, float z) { *p = (bf16_t)z; }
};
template <> struct VIo<float> {
    // fp32 logits are moved as float vectors: no bit casts of vector elements
    struct Raw { f32x4 a, b; };
    template <bool NT = false>
    __device__ static inline Raw load(const float *p) {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
        if constexpr (NT) return Raw{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1)};
        else return Raw{q[0], q[1]};
    }
    __device__ static inline void widen(const Raw &r, float z[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[k] = r.a[k];
            z[4 + k] = r.b[k];
        }
    }
    template <bool NT = false>
    __device__ static inline void store(float *p, const float z[8]) {
        const f32x4 a = {z[0], z[1], z[2], z[3]}, b = {z[4], z[5], z[6], z[7]};
        f32x4 *q = reinterpret_cast<f32x4 *>(p);
        if constexpr (NT) {
            __builtin_nontemporal_store(a, q);
            __builtin_nontemporal_store(b, q + 1);
        } else {
            q[0] = a;
            q[1] = b;
        }
    }
    __device__ static inline float load1(const float *p) { return *p; }
    __device__ static inline void store1(float *p, float z) { *p = z; }
};

// ---------------------------------------------------------------- row state
// Over the logits v a lane has seen, with c = log2(e) / T and raw references
// mt, ms (logit units):
//   lt = sum 2^(c (zt[v] - mt)),  d = sum 2^(c (zt[v] - mt)) (zt[v] - zs[v]),
//   ls = sum 2^(c (zs[v] - ms)).
// Finish: LSE_t = (c mt + log2 lt) ln 2, LSE_s likewise, and
//   KL = (d / lt) / T - LSE_t + LSE_s   (= E_p[zt/T - zs/T] - LSE_t + LSE_s).
struct VState {
    float mt, lt, d, ms, ls;
};

__device__ inline void vs_init(VState &s) {
    s.mt = kNoRef; s.lt = 0.f; s.d = 0.f; s.ms = kNoRef; s.ls = 0.f;
}

__device__ inline float max8(const float z[8]) {
    return fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
}

// Terms of one step under the current references: the step's sums of
// 2^(c (zt - mt)), 2^(c (zs - ms)) and 2^(c (zt - mt)) (zt - zs).
__device__ inline void step_terms(const VState &s, const float zt[8], const float zs[8], float c, float &lt,
                                  float &ls, float &d) {
    const float nt = -c * s.mt, ns = -c * s.ms;
    float lt0 = exp2_fast(fmaf(zt[0], c, nt)), lt1 = exp2_fast(fmaf(zt[1], c, nt));
    float ls0 = exp2_fast(fmaf(zs[0], c, ns)), ls1 = exp2_fast(fmaf(zs[1], c, ns));
    float d0 = lt0 * (zt[0] - zs[0]), d1 = lt1 * (zt[1] - zs[1]);
#pragma unroll
    for (int i = 2; i < 8; i += 2) {
        const float e0 = exp2_fast(fmaf(zt[i], c, nt)), e1 = exp2_fast(fmaf(zt[i + 1], c, nt));
        const float f0 = exp2_fast(fmaf(zs[i], c, ns)), f1 = exp2_fast(fmaf(zs[i + 1], c, ns));
        lt0 += e0; lt1 += e1;
        ls0 += f0; ls1 += f1;
        d0 = fmaf(e0, zt[i] - zs[i], d0);
        d1 = fmaf(e1, zt[i + 1] - zs[i + 1], d1);
    }
    lt = lt0 + lt1;
    ls = ls0 + ls1;
    d = d0 + d1;
}

// Fold 8 (teacher, student) logit pairs into the lane's state.  The step's
// terms are computed under the current references first; only if a sum
// exceeds 2^64 (some logit lies more than ~61 above its reference in the
// exponent, or the lane has no reference yet, which overflows to inf) are the
// references raised to the step's maxima and the terms computed again.  The
// check needs no per-step maximum on the common path.
__device__ inline void vs_fold8(VState &s, const float zt[8], const float zs[8], float c) {
    constexpr float kBig = 18446744073709551616.f;  // 2^64
    float lt, ls, d;
    step_terms(s, zt, zs, c, lt, ls, d);
    if (!(lt <= kBig) || !(ls <= kBig)) {  // rare: a lane's first step, or a far larger logit
        const float xt = fmaxf(s.mt, max8(zt)), xs = fmaxf(s.ms, max8(zs));
        const float w = exp2_fast(c * (s.mt - xt)), v = exp2_fast(c * (s.ms - xs));
        s.lt *= w;
        s.d *= w;
        s.ls *= v;
        s.mt = xt;
        s.ms = xs;
        step_terms(s, zt, zs, c, lt, ls, d);
    }
    s.lt += lt;
    s.ls += ls;
    s.d += d;
}

__device__ inline void vs_merge(VState &a, const VState &b, float c) {
    const float mt = fmaxf(a.mt, b.mt), ms = fmaxf(a.ms, b.ms);
    const float wa = exp2_fast(c * (a.mt - mt)), wb = exp2_fast(c * (b.mt - mt));
    const float va = exp2_fast(c * (a.ms - ms)), vb = exp2_fast(c * (b.ms - ms));
    a.lt = a.lt * wa + b.lt * wb;
    a.d = a.d * wa + b.d * wb;
    a.ls = a.ls * va + b.ls * vb;
    a.mt = mt;
    a.ms = ms;
}

__device__ inline VState vs_shfl_xor(const VState &s, int m) {
    VState o;
    o.mt = __shfl_xor(s.mt, m);
    o.lt = __shfl_xor(s.lt, m);
    o.d = __shfl_xor(s.d, m);
    o.ms = __shfl_xor(s.ms, m);
    o.ls = __shfl_xor(s.ls, m);
    return o;
}

struct VocabParams {
    const void *zt, *zs;
    int64_t rows, ld_t, ld_s;
    int V;
    float c;      // log2(e) / T
    float scale;  // 1 / T
    // forward outputs / backward inputs
    float *kl, *lse_t, *lse_s;
    // backward
    const float *g;
    float g_scalar;
    void *dzs, *dzt;
};

// Lane-subset pass of one row: the lane's state over its logits.
// LPR lanes share the row; `li` is this lane's index among them.
// Elements before the first 16-byte boundary of a row (p is element-aligned).
template <typename T> __device__ inline int head_elems(const T *p) {
    return (int)(((16u - ((unsigned)(uintptr_t)p & 15u)) & 15u) / sizeof(T));
}

// Vector steps over a 16-byte aligned run of n (a multiple of 8) logits.
template <typename T, int LPR, int kUnroll, bool NT>
__device__ inline void state_vec(const T *zt, const T *zs, int n, float c, int li, VState &s) {
    using Io = VIo<T>;
    const int nst = n / kStep;
    int k = li;
    for (; k + (kUnroll - 1) * LPR < nst; k += kUnroll * LPR) {
        typename Io::Raw a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            a[u] = Io::template load<NT>(zt + (int64_t)(k + u * LPR) * kStep);
            b[u] = Io::template load<NT>(zs + (int64_t)(k + u * LPR) * kStep);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float x[8], y[8];
            Io::widen(a[u], x);
            Io::widen(b[u], y);
            vs_fold8(s, x, y, c);
        }
    }
    for (; k < nst; k += LPR) {
        float x[8], y[8];
        Io::widen(Io::template load<NT>(zt + (int64_t)k * kStep), x);
        Io::widen(Io::template load<NT>(zs + (int64_t)k * kStep), y);
        vs_fold8(s, x, y, c);
    }
}

// Lane-subset pass of one row: the lane's state over its logits.
// LPR lanes share the row; `li` is this lane's index among them.  VEC: the
// row is 16-byte aligned and V a multiple of 8.  Otherwise, when both rows
// start equally far from a 16-byte boundary (always so for two contiguous
// [rows, V] matrices with aligned bases), lanes 0-7 take the head before the
// first boundary and lanes 8-15 the tail after the last whole step, one logit
// each, and the aligned body is streamed as in the vector case; rows without
// that match are read one logit per lane and step.
template <typename T, bool VEC, int LPR, bool NT, int kUnroll = kUnrollState>
__device__ inline void row_state(const T *zt, const T *zs, int V, float c, int li, VState &s) {
    using Io = VIo<T>;
    if (VEC) {
        state_vec<T, LPR, kUnroll, NT>(zt, zs, V, c, li, s);
        return;
    }
    const int h = head_elems(zt);
    if (h == head_elems(zs) && h <= V) {
        const int body = ((V - h) / kStep) * kStep;
        float x[8], y[8];
#pragma unroll
        for (int j = 1; j < 8; ++j) x[j] = y[j] = kPad;
        int v = -1;
        if (li < 8) v = li < h ? li : -1;
        else if (li < 16) v = h + body + (li - 8) < V ? h + body + (li - 8) : -1;
        x[0] = v >= 0 ? Io::load1(zt + v) : kPad;
        y[0] = v >= 0 ? Io::load1(zs + v) : kPad;
        vs_fold8(s, x, y, c);
        state_vec<T, LPR, kUnroll, NT>(zt + h, zs + h, body, c, li, s);
        return;
    }
    for (int base = 0; base < V; base += kStep * LPR) {
        float x[8], y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = base + li + j * LPR;
            const bool in = v < V;
            x[j] = in ? Io::load1(zt + v) : kPad;
            y[j] = in ? Io::load1(zs + v) : kPad;
        }
        vs_fold8(s, x, y, c);
    }
}

// Reduce the row's lane states so that EVERY lane of the row ends with the
// same merged state: an xor butterfly within each wave and lane 0's result
// broadcast to the wave (the lanes' results may differ in the last bit where
// a merge contracts to an fma); with WPR waves per row, each wave's state then
// goes through LDS and a second butterfly over WPR lanes (lane l reading wave
// l % WPR) combines them, again broadcast from lane 0.  red: LDS scratch of 5
// floats per wave.
__device__ inline void vs_bcast0(VState &s) {
    s.mt = __shfl(s.mt, 0); s.lt = __shfl(s.lt, 0); s.d = __shfl(s.d, 0);
    s.ms = __shfl(s.ms, 0); s.ls = __shfl(s.ls, 0);
}

template <int WPR>
__device__ inline void row_reduce(VState &s, float c, float *red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) vs_merge(s, vs_shfl_xor(s, m), c);
    vs_bcast0(s);
    if (WPR > 1) {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0) {
            red[wave * 5 + 0] = s.mt; red[wave * 5 + 1] = s.lt; red[wave * 5 + 2] = s.d;
            red[wave * 5 + 3] = s.ms; red[wave * 5 + 4] = s.ls;
        }
        __syncthreads();
        const int w = lane % WPR;
        s = VState{red[w * 5 + 0], red[w * 5 + 1], red[w * 5 + 2], red[w * 5 + 3], red[w * 5 + 4]};
#pragma unroll
        for (int m = WPR / 2; m >= 1; m >>= 1) vs_merge(s, vs_shfl_xor(s, m), c);
        vs_bcast0(s);
    }
}

struct RowResult {
    float kl, lt, ls;
};

__device__ inline RowResult row_finish(const VState &s, float c, float scale) {
    RowResult r;
    r.lt = (c * s.mt + log2_fast(s.lt)) * kLn2;
    r.ls = (c * s.ms + log2_fast(s.ls)) * kLn2;
    r.kl = (s.d / s.lt) * scale - r.lt + r.ls;
    return r;
}

// ================================================================= forward
template <typename T, bool VEC, int WPR>
__global__ __launch_bounds__(block_threads<WPR>()) void streamkl_vocab_fwd_kernel(VocabParams p) {
    constexpr int LPR = 64 * WPR;
    constexpr int RPB = rows_per_block<WPR>();
    __shared__ float red[(block_threads<WPR>() / 64) * 5];
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (WPR == 1 && row >= p.rows) return;  // whole waves only; no barrier below for WPR == 1
    const int li = threadIdx.x % LPR;
    const T *zt = static_cast<const T *>(p.zt) + row * p.ld_t;
    const T *zs = static_cast<const T *>(p.zs) + row * p.ld_s;
    VState s;
    vs_init(s);
    row_state<T, VEC, LPR, true>(zt, zs, p.V, p.c, li, s);
    row_reduce<WPR>(s, p.c, red);
    if (li == 0) {
        const RowResult r = row_finish(s, p.c, p.scale);
        p.kl[row] = r.kl;
        p.lse_t[row] = r.lt;
        p.lse_s[row] = r.ls;
    }
}

// ================================================================= backward
// dz_s[v] = g scale (q[v] - p[v]);  dz_t[v] = g scale p[v] (scale (zt - zs)[v] - (LSE_t - LSE_s) - KL)
// with p = 2^(c zt - LSE_t log2 e), q = 2^(c zs - LSE_s log2 e).
struct GradRow {
    float nlt, nls;  // -LSE log2(e)
    float gs;        // g / T
    float a, b;      // teacher: dz_t = p (a (zt - zs) + b)
};

template <bool TEACHER>
__device__ inline void grad8(const GradRow &r, float c, const float zt[8], const float zs[8], float dzs[8],
                             float dzt[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float pt = exp2_fast(fmaf(zt[i], c, r.nlt));
        const float ps = exp2_fast(fmaf(zs[i], c, r.nls));
        dzs[i] = r.gs * (ps - pt);
        if (TEACHER) dzt[i] = pt * fmaf(zt[i] - zs[i], r.a, r.b);
    }
}

template <bool TEACHER>
__device__ inline GradRow grad_row(const VocabParams &p, int64_t row, float kl, float lt, float ls) {
    GradRow r;
    const float g = p.g ? p.g[row] : p.g_scalar;
    r.gs = g * p.scale;
    r.nlt = -lt * kLog2e;
    r.nls = -ls * kLog2e;
    r.a = TEACHER ? r.gs * p.scale : 0.f;
    r.b = TEACHER ? -r.gs * (lt - ls + kl) : 0.f;
    return r;
}

// Vector steps of the gradient pass over a 16-byte aligned run of n (a
// multiple of 8) logits and the matching runs of the outputs.
// REV: walk the steps from the end of the run (the fused launch's second
// pass, so that it starts with the logits its first pass read last).
template <typename T, bool TEACHER, int LPR, int kUnroll, bool REV, bool NT>
__device__ inline void grads_vec(const GradRow &r, float c, const T *zt, const T *zs, T *gs_out, T *gt_out, int n,
                                 int li) {
    using Io = VIo<T>;
    const int nst = n / kStep;
    auto at = [&](int k) { return (int64_t)(REV ? nst - 1 - k : k) * kStep; };
    int k = li;
    for (; k + (kUnroll - 1) * LPR < nst; k += kUnroll * LPR) {
        typename Io::Raw a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            a[u] = Io::template load<NT>(zt + at(k + u * LPR));
            b[u] = Io::template load<NT>(zs + at(k + u * LPR));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float x[8], y[8], ds[8], dt[8];
            Io::widen(a[u], x);
            Io::widen(b[u], y);
            grad8<TEACHER>(r, c, x, y, ds, dt);
            Io::template store<NT>(gs_out + at(k + u * LPR), ds);
            if (TEACHER) Io::template store<NT>(gt_out + at(k + u * LPR), dt);
        }
    }
    for (; k < nst; k += LPR) {
        float x[8], y[8], ds[8], dt[8];
        Io::widen(Io::template load<NT>(zt + at(k)), x);
        Io::widen(Io::template load<NT>(zs + at(k)), y);
        grad8<TEACHER>(r, c, x, y, ds, dt);
        Io::template store<NT>(gs_out + at(k), ds);
        if (TEACHER) Io::template store<NT>(gt_out + at(k), dt);
    }
}

// Gradient pass of one row, with the same three layouts as row_state (the
// head/body/tail split also needs the output rows to start equally far from a
// 16-byte boundary).
template <typename T, bool VEC, bool TEACHER, int LPR, bool NT, int kUnroll = unroll_grad<T>(), bool REV = false>
__device__ inline void row_grads(const VocabParams &p, int64_t row, const GradRow &r, int li) {
    using Io = VIo<T>;
    const T *zt = static_cast<const T *>(p.zt) + row * p.ld_t;
    const T *zs = static_cast<const T *>(p.zs) + row * p.ld_s;
    T *gs_out = static_cast<T *>(p.dzs) + row * (int64_t)p.V;
    T *gt_out = TEACHER ? static_cast<T *>(p.dzt) + row * (int64_t)p.V : nullptr;
    const int V = p.V;
    if (VEC) {
        grads_vec<T, TEACHER, LPR, kUnroll, REV, NT>(r, p.c, zt, zs, gs_out, gt_out, V, li);
        return;
    }
    const int h = head_elems(zt);
    if (h == head_elems(zs) && h == head_elems(gs_out) && (!TEACHER || h == head_elems(gt_out)) && h <= V) {
        const int body = ((V - h) / kStep) * kStep;
        int v = -1;
        if (li < 8) v = li < h ? li : -1;
        else if (li < 16) v = h + body + (li - 8) < V ? h + body + (li - 8) : -1;
        if (v >= 0) {
            float x[8], y[8], ds[8], dt[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = y[j] = 0.f;
            x[0] = Io::load1(zt + v);
            y[0] = Io::load1(zs + v);
            grad8<TEACHER>(r, p.c, x, y, ds, dt);
            Io::store1(gs_out + v, ds[0]);
            if (TEACHER) Io::store1(gt_out + v, dt[0]);
        }
        grads_vec<T, TEACHER, LPR, kUnroll, REV, NT>(r, p.c, zt + h, zs + h, gs_out + h, TEACHER ? gt_out + h : nullptr,
                                                 body, li);
        return;
    }
    for (int base = 0; base < V; base += kStep * LPR) {
        float x[8], y[8], ds[8], dt[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = base + li + j * LPR;
            const bool in = v < V;
            x[j] = in ? Io::load1(zt + v) : 0.f;
            y[j] = in ? Io::load1(zs + v) : 0.f;
        }
        grad8<TEACHER>(r, p.c, x, y, ds, dt);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = base + li + j * LPR;
            if (v < V) {
                Io::store1(gs_out + v, ds[j]);
                if (TEACHER) Io::store1(gt_out + v, dt[j]);
            }
        }
    }
}

template <typename T, bool VEC, bool TEACHER, int WPR>
__global__ __launch_bounds__(block_threads<WPR>()) void streamkl_vocab_bwd_kernel(VocabParams p) {
    constexpr int LPR = 64 * WPR;
    constexpr int RPB = rows_per_block<WPR>();
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (row >= p.rows) return;  // no barrier in this kernel
    const GradRow r = grad_row<TEACHER>(p, row, TEACHER ? p.kl[row] : 0.f, p.lse_t[row], p.lse_s[row]);
    row_grads<T, VEC, TEACHER, LPR, true>(p, row, r, threadIdx.x % LPR);
}

// ================================================================= fused forward + backward
// The forward pass of a row, then, with the row's LSEs and KL known to every
// lane, the gradient pass over the same row (whose logits the first pass has
// just brought through the caches).
template <typename T, bool VEC, bool TEACHER, int WPR>
__global__ __launch_bounds__(block_threads<WPR>()) void streamkl_vocab_fused_kernel(VocabParams p) {
    constexpr int LPR = 64 * WPR;
    constexpr int RPB = rows_per_block<WPR>();
    __shared__ float red[(block_threads<WPR>() / 64) * 5];
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (WPR == 1 && row >= p.rows) return;  // no barrier below for WPR == 1
    const int li = threadIdx.x % LPR;
    const T *zt = static_cast<const T *>(p.zt) + row * p.ld_t;
    const T *zs = static_cast<const T *>(p.zs) + row * p.ld_s;
    VState s;
    vs_init(s);
    row_state<T, VEC, LPR, false>(zt, zs, p.V, p.c, li, s);  // ordinary loads: the second pass re-reads the row
    row_reduce<WPR>(s, p.c, red);  // every lane of the row holds the row's state
    const RowResult r = row_finish(s, p.c, p.scale);
    if (li == 0) {
        p.kl[row] = r.kl;
        p.lse_t[row] = r.lt;
        p.lse_s[row] = r.ls;
    }
    const GradRow gr = grad_row<TEACHER>(p, row, r.kl, r.lt, r.ls);
    // second pass from the end of the row: the logits read last are the likeliest still cached
    row_grads<T, VEC, TEACHER, LPR, true, kUnrollState, true>(p, row, gr, li);
}

// ================================================================= host side
#ifndef STREAMKL_VOCAB_WPR
#define STREAMKL_VOCAB_WPR 0  // nonzero: waves per row for every row of >= 4096 logits
#endif

enum Mode { kFwd, kBwd, kFused };

// Waves per row.  Short rows (< 4096 logits): one wave, four rows per
// workgroup.  Longer rows: one workgroup per row, of 8 waves for the forward
// and 16 for the backward and the fused launch (measured on 4096 x 128256
// bf16 rows; with 16 waves a CU holds a single row, so the fused launch has
// the fewest rows in flight and its second pass finds more of them in the
// caches).
int choose_wpr(Mode mode, int V) {
    if (V < 4096) return 1;
    if (STREAMKL_VOCAB_WPR) return STREAMKL_VOCAB_WPR;
    return mode == kFwd ? 8 : 16;
}

bool vec_ok(const void *p, int64_t ld, int V) {
    return ((uintptr_t)p) % 16 == 0 && (ld % kStep) == 0 && (V % kStep) == 0;
}

template <typename T, bool VEC, bool TEACHER, int WPR>
void launch_vocab(Mode mode, const VocabParams &p, unsigned grid, hipStream_t s) {
    const dim3 blk(block_threads<WPR>());
    if (mode == kFwd)
        hipLaunchKernelGGL((streamkl_vocab_fwd_kernel<T, VEC, WPR>), dim3(grid), blk, 0, s, p);
    else if (mode == kBwd)
        hipLaunchKernelGGL((streamkl_vocab_bwd_kernel<T, VEC, TEACHER, WPR>), dim3(grid), blk, 0, s, p);
    else
        hipLaunchKernelGGL((streamkl_vocab_fused_kernel<T, VEC, TEACHER, WPR>), dim3(grid), blk, 0, s, p);
}

typedef void (*vocab_launch_t)(Mode, const VocabParams &, unsigned, hipStream_t);

template <typename T, bool VEC, bool TEACHER>
vocab_launch_t pick_wpr(int wpr) {
    switch (wpr) {
        case 1: return launch_vocab<T, VEC, TEACHER, 1>;
        case 4: return launch_vocab<T, VEC, TEACHER, 4>;
        case 8: return launch_vocab<T, VEC, TEACHER, 8>;
        default: return launch_vocab<T, VEC, TEACHER, 16>;
    }
}

template <typename T>
vocab_launch_t pick_vocab(bool vec, bool teacher, int wpr) {
    if (vec) return teacher ? pick_wpr<T, true, true>(wpr) : pick_wpr<T, true, false>(wpr);
    return teacher ? pick_wpr<T, false, true>(wpr) : pick_wpr<T, false, false>(wpr);
}

streamkl_status vocab_check(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                            int64_t ld_t, int64_t ld_s, float temperature) {
    if (!z_t || !z_s) return STREAMKL_ERR_INVALID;
    if (dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) return STREAMKL_ERR_INVALID;
    if (rows < 1 || V < 1 || V > (1 << 30)) return STREAMKL_ERR_INVALID;
    if (ld_t < V || ld_s < V) return STREAMKL_ERR_INVALID;
    if (!(temperature >= 1e-4f && temperature <= 1e6f)) return STREAMKL_ERR_INVALID;
    const int elt = dtype == STREAMKL_BF16 ? 2 : 4;
    if (((uintptr_t)z_t) % elt != 0 || ((uintptr_t)z_s) % elt != 0) return STREAMKL_ERR_INVALID;
    // row offsets of the launches stay within the address space
    if (rows > INT64_MAX / 8 / (ld_t > ld_s ? ld_t : ld_s)) return STREAMKL_ERR_INVALID;
    return STREAMKL_OK;
}

// Rows per launch: a dispatch holds fewer than 2^32 work-items (64 WPR per row).
constexpr int64_t kRowsPerLaunch = 1 << 20;

streamkl_status vocab_launch(Mode mode, const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                             int64_t ld_t, int64_t ld_s, float temperature, float *kl, float *lse_t, float *lse_s,
                             const float *grad_rows, float grad_scalar, void *dz_s, void *dz_t, void *stream) {
    const int elt = dtype == STREAMKL_BF16 ? 2 : 4;
    bool vec = vec_ok(z_t, ld_t, V) && vec_ok(z_s, ld_s, V);
    if (mode != kFwd) vec = vec && vec_ok(dz_s, V, V) && (!dz_t || vec_ok(dz_t, V, V));
    const int wpr = choose_wpr(mode, V);
    const vocab_launch_t fn = dtype == STREAMKL_BF16 ? pick_vocab<bf16_t>(vec, dz_t != nullptr, wpr)
                                                     : pick_vocab<float>(vec, dz_t != nullptr, wpr);
    const int rpb = wpr == 1 ? 4 : 1;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (streamkl_internal::log_enabled())
        fprintf(stderr,
                "[streamkl] vocab %s %s rows=%lld V=%d: %d wave(s) per row, %d row(s) per block, %s loads, "
                "%lld launch(es) of up to %lld rows\n",
                mode == kFwd ? "fwd" : (mode == kBwd ? "bwd" : "fused"), dtype == STREAMKL_BF16 ? "bf16" : "f32",
                (long long)rows, V, wpr, rpb, vec ? "16-byte" : "element", (long long)((rows + kRowsPerLaunch - 1) / kRowsPerLaunch),
                (long long)kRowsPerLaunch);
    for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
        const int64_t n = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
        VocabParams p{};
        p.zt = static_cast<const char *>(z_t) + r0 * ld_t * elt;
        p.zs = static_cast<const char *>(z_s) + r0 * ld_s * elt;
        p.rows = n; p.ld_t = ld_t; p.ld_s = ld_s; p.V = V;
        p.scale = 1.0f / temperature;
        p.c = kLog2e / temperature;
        p.kl = kl ? kl + r0 : nullptr;
        p.lse_t = lse_t + r0;
        p.lse_s = lse_s + r0;
        p.g = grad_rows ? grad_rows + r0 : nullptr;
        p.g_scalar = grad_scalar;
        p.dzs = dz_s ? static_cast<char *>(dz_s) + r0 * (int64_t)V * elt : nullptr;
        p.dzt = dz_t ? static_cast<char *>(dz_t) + r0 * (int64_t)V * elt : nullptr;
        fn(mode, p, (unsigned)((n + rpb - 1) / rpb), hs);
        if (hipGetLastError() != hipSuccess) return STREAMKL_ERR_HIP;
    }
    return STREAMKL_OK;
}

bool grad_ptrs_ok(const void *dz_s, const void *dz_t, int elt) {
    if (!dz_s || ((uintptr_t)dz_s) % elt != 0) return false;
    if (dz_t && ((uintptr_t)dz_t) % elt != 0) return false;
    return true;
}

}  // namespace

extern "C" {

streamkl_status streamkl_vocab_fwd(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                                   int64_t ld_t, int64_t ld_s, float temperature, float *kl_rows, float *lse_t,
                                   float *lse_s, float *kl_sum, void *stream) {
    streamkl_status rc = vocab_check(z_t, z_s, dtype, rows, V, ld_t, ld_s, temperature);
    if (rc != STREAMKL_OK) return rc;
    if (!kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    rc = vocab_launch(kFwd, z_t, z_s, dtype, rows, V, ld_t, ld_s, temperature, kl_rows, lse_t, lse_s, nullptr, 0.f,
                      nullptr, nullptr, stream);
    if (rc != STREAMKL_OK) return rc;
    if (kl_sum && streamkl_internal::launch_row_sum(kl_rows, rows, kl_sum, static_cast<hipStream_t>(stream)) !=
                      hipSuccess)
        return STREAMKL_ERR_HIP;
    return STREAMKL_OK;
}

streamkl_status streamkl_vocab_bwd(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                                   int64_t ld_t, int64_t ld_s, float temperature, const float *lse_t,
                                   const float *lse_s, const float *kl_rows, const float *grad_rows,
                                   float grad_scalar, void *dz_s, void *dz_t, void *stream) {
    streamkl_status rc = vocab_check(z_t, z_s, dtype, rows, V, ld_t, ld_s, temperature);
    if (rc != STREAMKL_OK) return rc;
    if (!lse_t || !lse_s || (dz_t && !kl_rows)) return STREAMKL_ERR_INVALID;
    if (!grad_ptrs_ok(dz_s, dz_t, dtype == STREAMKL_BF16 ? 2 : 4)) return STREAMKL_ERR_INVALID;
    return vocab_launch(kBwd, z_t, z_s, dtype, rows, V, ld_t, ld_s, temperature, const_cast<float *>(kl_rows),
                        const_cast<float *>(lse_t), const_cast<float *>(lse_s), grad_rows, grad_scalar, dz_s, dz_t,
                        stream);
}

streamkl_status streamkl_vocab_fwd_bwd(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                                       int64_t ld_t, int64_t ld_s, float temperature, const float *grad_rows,
                                       float grad_scalar, float *kl_rows, float *lse_t, float *lse_s,
                                       float *kl_sum, void *dz_s, void *dz_t, void *stream) {
    streamkl_status rc = vocab_check(z_t, z_s, dtype, rows, V, ld_t, ld_s, temperature);
    if (rc != STREAMKL_OK) return rc;
    if (!kl_rows || !lse_t || !lse_s) return STREAMKL_ERR_INVALID;
    if (!grad_ptrs_ok(dz_s, dz_t, dtype == STREAMKL_BF16 ? 2 : 4)) return STREAMKL_ERR_INVALID;
    rc = vocab_launch(kFused, z_t, z_s, dtype, rows, V, ld_t, ld_s, temperature, kl_rows, lse_t, lse_s, grad_rows,
                      grad_scalar, dz_s, dz_t, stream);
    if (rc != STREAMKL_OK) return rc;
    if (kl_sum && streamkl_internal::launch_row_sum(kl_rows, rows, kl_sum, static_cast<hipStream_t>(stream)) !=
                      hipSuccess)
        return STREAMKL_ERR_HIP;
    return STREAMKL_OK;
}

}  // extern "C"
