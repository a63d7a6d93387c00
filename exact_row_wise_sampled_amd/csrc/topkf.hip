// Exact FP32 row-wise Top-K for MI355X (gfx950): a sample-guided exact
// selector after "Sample-Guided Exact Top-K Selection for Long-Context Sparse
// Attention" (Secs. 4-5), behind the C ABI declared in include/topkf.h.
//
// One 512-thread workgroup (8 wave64) works on a row at a time:
//   Phase 1 (Sec. 4.2, Eqs. 11-15; Sec. 5.2): the regular view
//     V = {i < L : i = a_r mod s} is projected to the 11-bit coarse key and
//     histogrammed in LDS; the first bins whose prefix reaches q = ceil(1.5K/s)
//     and q1 = ceil(1.75K/s) give tau0 and tau1, converted once to inclusive
//     FP32 cutoffs expressed as descending integer keys.
//   Phase 2 (Sec. 4.3, Eqs. 16-17; Sec. 5.3): one streaming pass over the
//     row with 128-bit nontemporal loads admits key <= T0, appends the
//     (index, key) pair to the frontier and counts its leading 11-bit digit.
//     Underfill (C < K) appends the band T0 < key <= T1 in a second pass
//     (Eqs. 18-19); continued underfill, an unusable view or the no-view
//     policy take the exact coarse route (Eq. 20).
//   Phase 3 (Sec. 4.4, Eqs. 22-25; Sec. 5.4): 11+11+10-bit refinement of the
//     FP32 descending key over the frontier only, through two ping-pong
//     buffers (LDS first, then a global spill slice).
// Two mappings (Sec. 4.5, Sec. 5.5): a persistent pool whose workgroups take
// rows from a device queue, and a KV-split mapping in which P workgroups scan
// disjoint segments of one row and the last to arrive finishes it.
//
// Every wave of a workgroup runs the same trip counts, so the ballots below
// always see all 64 lanes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "topkf.h"

namespace {

constexpr int kBlock = 512;
constexpr int kWaves = kBlock / 64;
constexpr int kBins = 2048;
constexpr int kCapA = 4096;  // LDS frontier A (Q0, Q2), (index, key) pairs
constexpr int kCapB = 2048;  // LDS frontier B (Q1)
constexpr int kUnroll = 4;   // 128-bit loads in flight per thread
// A NaN pattern whose descending key is 0xFFFFFFFF: larger than every cutoff,
// so it marks lanes that hold no element.
constexpr uint32_t kNoElem = 0xFFFFFFFFu;
constexpr uint32_t kKeyFirst = 0x007FFFFFu;  // descending key of +inf
constexpr uint32_t kKeyLast = 0xFF800000u;   // descending key of -inf

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Params {
    const float* logits;
    int64_t stride;
    const int32_t* ke;
    int32_t* out;
    const int32_t* num_valid_rows;
    uint32_t* counters;
    uint2* ws;
    uint32_t* stats;
    int32_t m_cap;
    int32_t n;
    int32_t k;
    int32_t splits;
    int32_t min_seg;
};

struct alignas(16) Shared {
    uint32_t hist[2][kBins];
    uint2 qa[kCapA];
    uint2 qb[kCapB];
    uint32_t wsum[kWaves];
    uint32_t res[4];
    uint32_t cnt[2];
    uint32_t out_cnt;
    uint32_t tie_cnt;
    uint32_t cut[2];
    int32_t next_row;
    uint32_t flag;
};
static_assert(sizeof(Shared) <= 80 * 1024, "two workgroups per CU must fit in LDS");

// ------------------------------------------------------------------ keys

// Descending sortable key of an FP32 bit pattern: a larger value gets a
// smaller key (+inf -> 0x007FFFFF, +0 -> 0x7FFFFFFF, -0 -> 0x80000000,
// -inf -> 0xFF800000); the order refines the numeric order with +0 above -0.
__device__ __forceinline__ uint32_t desc_key(uint32_t b) {
    return b ^ ((~static_cast<uint32_t>(static_cast<int32_t>(b) >> 31)) >> 1);
}

__device__ __forceinline__ uint32_t bits_of_key(uint32_t k) {
    return k <= 0x7FFFFFFFu ? (k ^ 0x7FFFFFFFu) : k;
}

// Sec. 4.2, Eq. 11: c(x) = kappa16(fp16_rne(x)) >> 5 in [0, 2048).
__device__ __forceinline__ uint32_t coarse_of_bits(uint32_t b) {
    const _Float16 h = static_cast<_Float16>(__uint_as_float(b));
    const uint32_t hb = static_cast<uint32_t>(__builtin_bit_cast(unsigned short, h));
    const uint32_t k16 = (hb & 0x8000u) ? hb : (hb ^ 0x7FFFu);
    return k16 >> 5;
}

// Sec. 4.3: the inclusive FP32 cutoff of coarse bin tau, as the largest
// non-NaN descending key whose value still has c <= tau.  c is monotone in the
// key, so {c(x) <= tau} == {key(x) <= cutoff(tau)}.  Returns kKeyFirst - 1
// (admits no non-NaN value) when even +inf lies above tau.
__device__ uint32_t cutoff_key(uint32_t tau) {
    if (coarse_of_bits(bits_of_key(kKeyFirst)) > tau) return kKeyFirst - 1;
    if (coarse_of_bits(bits_of_key(kKeyLast)) <= tau) return kKeyLast;
    uint32_t lo = kKeyFirst, hi = kKeyLast;  // c(lo) <= tau < c(hi)
    while (hi - lo > 1) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (coarse_of_bits(bits_of_key(mid)) <= tau) lo = mid; else hi = mid;
    }
    return lo;
}

// Refinement digit j of a descending key: 11 + 11 + 10 bits, most
// significant first (Sec. 4.3 "D = 3 digits of widths 11 + 11 + 10").
__device__ __forceinline__ uint32_t digit(int j, uint32_t key) {
    return j == 0 ? (key >> 21) : (j == 1 ? ((key >> 10) & 0x7FFu) : (key & 0x3FFu));
}

// Row phase a_r = pi_s(r mod s) (Sec. 4.2, Eq. 13): pi_s reverses the
// log2(s) bits, so each block of s consecutive rows uses every residue once.
__device__ __forceinline__ uint32_t view_phase(uint32_t row, int s) {
    const int bitsn = s == 128 ? 7 : 6;
    return __builtin_bitreverse32(row & (s - 1)) >> (32 - bitsn);
}

// ------------------------------------------------------------ wave helpers

__device__ __forceinline__ uint32_t lane() { return __lane_id(); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, uint64_t m, uint32_t n) {
    const int leader = __builtin_ctzll(m);
    uint32_t base = 0;
    if (static_cast<int>(lane()) == leader) base = atomicAdd(counter, n);
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), leader));
}

__device__ __forceinline__ void lds_inc(uint32_t* h, uint32_t bin) {
    __hip_atomic_fetch_add(h + bin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------- frontier

// Entries [0, cap) live in LDS, entries [cap, count) in a global slice.
struct Frontier {
    uint2* lds;
    uint32_t cap;
    uint2* gbl;
    uint32_t* cnt;  // LDS counter
};

__device__ __forceinline__ void fput(const Frontier& f, uint32_t slot, uint2 item) {
    if (slot < f.cap) f.lds[slot] = item; else f.gbl[slot - f.cap] = item;
}

__device__ __forceinline__ uint2 fget(const Frontier& f, uint32_t e) {
    return e < f.cap ? f.lds[e] : f.gbl[e - f.cap];
}

// Output commit: lanes with `pred` take the next output slots.
__device__ __forceinline__ void commit(bool pred, uint32_t idx, int32_t* outp, uint32_t k,
                                       Shared& sm) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return;
    const uint32_t base = wave_reserve(&sm.out_cnt, m, __builtin_popcountll(m));
    if (pred) {
        const uint32_t slot = base + mbcnt(m);
        if (slot < k) outp[slot] = static_cast<int32_t>(idx);
    }
}

// Frontier append of (idx, key) with a histogram count of `bin` in `h`.
__device__ __forceinline__ void append(bool pred, uint32_t idx, uint32_t key, uint32_t bin,
                                       const Frontier& f, uint32_t* h) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return;
    const uint32_t base = wave_reserve(f.cnt, m, __builtin_popcountll(m));
    if (pred) {
        fput(f, base + mbcnt(m), make_uint2(idx, key));
        lds_inc(h, bin);
    }
}

// ------------------------------------------------------------ block scan

// For each target t[i] (1 <= t[i] <= sum of hist), finds b = min{b : H(b) >=
// t[i]} and H(b - 1) (Eqs. 15, 23), written to sm.res[2i], sm.res[2i + 1].
// Each thread owns 4 consecutive bins.  Reads hist before its first barrier
// and ends with a barrier, so hist may be rewritten right after it returns.
template <int NT>
__device__ void block_find(const uint32_t* hist, const uint32_t (&t)[NT], Shared& sm) {
    const int tid = threadIdx.x;
    // Defaults keep every later LDS index in range should a target exceed
    // the histogram total (only possible for NaN inputs, which the contract
    // excludes); the finding thread overwrites them after the first barrier.
    if (tid == 0) {
#pragma unroll
        for (int i = 0; i < NT; ++i) { sm.res[2 * i] = kBins - 1; sm.res[2 * i + 1] = 0; }
    }
    const uint4 v = reinterpret_cast<const uint4*>(hist)[tid];
    const uint32_t s = v.x + v.y + v.z + v.w;
    uint32_t incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (static_cast<int>(lane()) >= d) incl += o;
    }
    if (lane() == 63) sm.wsum[tid >> 6] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < (tid >> 6); ++w) base += sm.wsum[w];
    const uint32_t excl = base + incl - s;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (excl < t[i] && t[i] <= excl + s) {
            uint32_t acc = excl, b = 4 * tid;
            if (acc + v.x < t[i]) {
                acc += v.x; b += 1;
                if (acc + v.y < t[i]) {
                    acc += v.y; b += 1;
                    if (acc + v.z < t[i]) { acc += v.z; b += 1; }
                }
            }
            sm.res[2 * i] = b;
            sm.res[2 * i + 1] = acc;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void clear_hist(uint32_t* h) {
    reinterpret_cast<uint4*>(h)[threadIdx.x] = make_uint4(0, 0, 0, 0);
}

// ------------------------------------------------------------- streaming

// Calls f(bits4, index_of_bits4.x) over elements [lo, hi) of row x: 128-bit
// nontemporal loads for the 16-byte aligned body, one element per lane for
// the unaligned head and the tail.  Lanes without an element see kNoElem.
// Every thread of the block must call it with the same arguments.
template <class F>
__device__ __forceinline__ void stream_range(const float* x, uint32_t lo, uint32_t hi, F&& f) {
    if (hi <= lo) return;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(x + lo);
    uint32_t head = static_cast<uint32_t>(((16u - (addr & 15u)) & 15u) >> 2);
    if (head > hi - lo) head = hi - lo;
    const uint32_t vlo = lo + head;
    const uint32_t nvec = (hi - vlo) >> 2;
    const uint32_t tlo = vlo + 4 * nvec;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x + vlo);
    const uint32_t tid = threadIdx.x;
    for (uint32_t base = 0; base < nvec; base += kBlock * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t vi = base + u * kBlock + tid;
            if (vi < nvec) v[u] = __builtin_nontemporal_load(xv + vi);
            else v[u] = u32x4{kNoElem, kNoElem, kNoElem, kNoElem};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) f(v[u], vlo + 4 * (base + u * kBlock + tid));
    }
    const uint32_t nscal = head + (hi - tlo);
    if (nscal) {
        const uint32_t e = tid < head ? lo + tid : tlo + (tid - head);
        const uint32_t b = tid < nscal ? __float_as_uint(x[e]) : kNoElem;
        f(u32x4{b, kNoElem, kNoElem, kNoElem}, e);
    }
}

// Phase 2 admission of one 4-element group: key <= hi (and key > lo for the
// band pass of Eq. 18), appended to frontier f with its leading digit counted
// in h (Eq. 17).  One LDS reservation per wave and group.
template <bool BAND>
__device__ __forceinline__ void admit4(u32x4 b, uint32_t i0, uint32_t klo, uint32_t khi,
                                       const Frontier& f, uint32_t* h) {
    const uint32_t k0 = desc_key(b.x), k1 = desc_key(b.y), k2 = desc_key(b.z), k3 = desc_key(b.w);
    const bool p0 = k0 <= khi && (!BAND || k0 > klo);
    const bool p1 = k1 <= khi && (!BAND || k1 > klo);
    const bool p2 = k2 <= khi && (!BAND || k2 > klo);
    const bool p3 = k3 <= khi && (!BAND || k3 > klo);
    const uint64_t m0 = __ballot(p0), m1 = __ballot(p1), m2 = __ballot(p2), m3 = __ballot(p3);
    const uint64_t any = m0 | m1 | m2 | m3;
    if (any == 0) return;
    const uint32_t c0 = __builtin_popcountll(m0), c1 = __builtin_popcountll(m1);
    const uint32_t c2 = __builtin_popcountll(m2), c3 = __builtin_popcountll(m3);
    uint32_t base = wave_reserve(f.cnt, any, c0 + c1 + c2 + c3);
    if (p0) { fput(f, base + mbcnt(m0), make_uint2(i0, k0)); lds_inc(h, k0 >> 21); }
    base += c0;
    if (p1) { fput(f, base + mbcnt(m1), make_uint2(i0 + 1, k1)); lds_inc(h, k1 >> 21); }
    base += c1;
    if (p2) { fput(f, base + mbcnt(m2), make_uint2(i0 + 2, k2)); lds_inc(h, k2 >> 21); }
    base += c2;
    if (p3) { fput(f, base + mbcnt(m3), make_uint2(i0 + 3, k3)); lds_inc(h, k3 >> 21); }
}

// ------------------------------------------------------------ row pieces

__device__ void sentinel_row(int32_t* outp, uint32_t L, uint32_t k) {
    for (uint32_t j = threadIdx.x; j < k; j += kBlock) outp[j] = j < L ? static_cast<int32_t>(j) : -1;
}

__device__ __forceinline__ void count_route(const Params& p, int route) {
    if (p.stats && threadIdx.x == 0) atomicAdd(p.stats + route, 1u);
}

// Phase 1: coarse histogram of the view into h (already cleared and visible),
// then tau0/tau1 and their cutoffs into sm.cut.  Ends with a barrier.
__device__ void phase1(const float* x, uint32_t a, uint32_t nv, int s, uint32_t q, uint32_t q1,
                       uint32_t* h, Shared& sm) {
    for (uint32_t j = threadIdx.x; j < nv; j += kBlock)
        lds_inc(h, coarse_of_bits(__float_as_uint(x[a + j * s])));
    __syncthreads();
    const uint32_t t[2] = {q, q1};
    block_find<2>(h, t, sm);
    if (threadIdx.x == 0) {
        const uint32_t tau0 = sm.res[0], tau1 = sm.res[2];
        sm.cut[0] = cutoff_key(tau0);
        sm.cut[1] = tau1 > tau0 ? cutoff_key(tau1) : sm.cut[0];
    }
    __syncthreads();
}

// Exact coarse route (Sec. 4.3, Eq. 20) over [0, L): coarse histogram of
// every value, tau* = min{b : C(b) >= K}, then one classification pass that
// commits c < tau* to the output and retains c == tau* in frontier A with its
// leading-digit histogram in h0.  Returns k0 = K - |E0|.
__device__ uint32_t exact_route(const float* x, uint32_t L, uint32_t k, int32_t* outp,
                                const Frontier& A, uint32_t* hc, uint32_t* h0, Shared& sm) {
    __syncthreads();  // earlier readers of the frontier count and histograms are done
    clear_hist(hc);
    clear_hist(h0);
    if (threadIdx.x == 0) { *A.cnt = 0; sm.out_cnt = 0; }
    __syncthreads();
    stream_range(x, 0, L, [&](u32x4 b, uint32_t) {
        if (b.x != kNoElem) lds_inc(hc, coarse_of_bits(b.x));
        if (b.y != kNoElem) lds_inc(hc, coarse_of_bits(b.y));
        if (b.z != kNoElem) lds_inc(hc, coarse_of_bits(b.z));
        if (b.w != kNoElem) lds_inc(hc, coarse_of_bits(b.w));
    });
    __syncthreads();
    const uint32_t t[1] = {k};
    block_find<1>(hc, t, sm);
    const uint32_t tau = sm.res[0], before = sm.res[1];
    stream_range(x, 0, L, [&](u32x4 b, uint32_t i0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t bc = b[c];
            const bool valid = bc != kNoElem;
            const uint32_t cc = coarse_of_bits(bc);
            commit(valid && cc < tau, i0 + c, outp, k, sm);
            const uint32_t key = desc_key(bc);
            append(valid && cc == tau, i0 + c, key, key >> 21, A, h0);
        }
    });
    __syncthreads();
    return k - before;
}

// Phase 3 (Sec. 4.4): refinement of frontier `cur` whose leading-digit
// histogram is in hc, with remaining quota kq.  Frontier counts and hc must
// be visible (barrier done).  Commits exactly kq more indices.
__device__ void refine(Frontier cur, Frontier nxt, uint32_t* hc, uint32_t* hn, uint32_t kq,
                       int32_t* outp, uint32_t k, Shared& sm) {
    const uint32_t tid = threadIdx.x;
    for (int j = 0; j < 3; ++j) {
        const uint32_t n = *cur.cnt;
        if (j < 2) clear_hist(hn);
        if (tid == 0) { *nxt.cnt = 0; sm.tie_cnt = 0; }
        const uint32_t t[1] = {kq};
        block_find<1>(hc, t, sm);
        const uint32_t b = sm.res[0], before = sm.res[1];
        const uint32_t inb = hc[b];
        const bool exact_fill = before + inb == kq;  // the boundary group fits exactly
        const bool last = exact_fill || j == 2;
        const uint32_t need = kq - before;
        for (uint32_t e0 = 0; e0 < n; e0 += kBlock) {
            const uint32_t e = e0 + tid;
            const bool valid = e < n;
            const uint2 it = valid ? fget(cur, e) : make_uint2(0u, 0u);
            const uint32_t d = digit(j, it.y);
            if (last) {
                bool take = valid && (exact_fill ? d <= b : d < b);
                if (!exact_fill) {
                    const bool tie = valid && d == b;
                    const uint64_t m = __ballot(tie);
                    if (m) {
                        const uint32_t base = wave_reserve(&sm.tie_cnt, m, __builtin_popcountll(m));
                        if (tie && base + mbcnt(m) < need) take = true;
                    }
                }
                commit(take, it.x, outp, k, sm);
            } else {
                commit(valid && d < b, it.x, outp, k, sm);
                append(valid && d == b, it.x, it.y, digit(j + 1, it.y), nxt, hn);
            }
        }
        __syncthreads();
        if (last) break;
        kq = need;
        const Frontier tf = cur; cur = nxt; nxt = tf;
        uint32_t* th = hc; hc = hn; hn = th;
    }
}

// Number of view samples and the view's phase for a row.
template <int S>
__device__ __forceinline__ uint32_t view_size(uint32_t row, uint32_t L, uint32_t* a) {
    *a = view_phase(row, S);
    return L > *a ? (L - *a + S - 1) / S : 0u;
}

__device__ __forceinline__ uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// q = ceil(K~/s) with K~ = ceil(1.5K), q1 with K~1 = ceil(1.75K) (Sec. 4.2;
// Sec. 6.4 "Conditional rescue").
__device__ __forceinline__ uint32_t q_primary(uint32_t k, int s) { return ceil_div(ceil_div(3 * k, 2), s); }
__device__ __forceinline__ uint32_t q_secondary(uint32_t k, int s) { return ceil_div(ceil_div(7 * k, 4), s); }

// One row, whole-row ownership (persistent mapping).
template <int S, bool DUAL>
__device__ void select_row(const Params& p, int row, Shared& sm, const Frontier& A,
                           const Frontier& B) {
    const uint32_t k = p.k;
    int32_t* outp = p.out + static_cast<int64_t>(row) * k;
    int32_t Ls = p.ke[row];
    const uint32_t L = static_cast<uint32_t>(Ls < 0 ? 0 : (Ls > p.n ? p.n : Ls));
    if (L <= k) {
        sentinel_row(outp, L, k);
        count_route(p, TOPKF_ROUTE_SENTINEL);
        return;
    }
    const float* x = p.logits + static_cast<int64_t>(row) * p.stride;
    uint32_t* h0 = sm.hist[0];
    uint32_t* h1 = sm.hist[1];
    int route = TOPKF_ROUTE_EXACT_DIRECT;
    bool certified = false;
    if constexpr (S > 0) {
        uint32_t a;
        const uint32_t nv = view_size<S>(row, L, &a);
        const uint32_t q = q_primary(k, S), q1 = DUAL ? q_secondary(k, S) : q;
        if (nv >= q1) {
            clear_hist(h0);
            clear_hist(h1);
            if (threadIdx.x == 0) { *A.cnt = 0; sm.out_cnt = 0; }
            __syncthreads();
            phase1(x, a, nv, S, q, q1, h0, sm);
            const uint32_t T0 = sm.cut[0], T1 = sm.cut[1];
            stream_range(x, 0, L, [&](u32x4 b, uint32_t i0) { admit4<false>(b, i0, 0u, T0, A, h1); });
            __syncthreads();
            uint32_t C = *A.cnt;
            route = TOPKF_ROUTE_PRIMARY;
            if (C < k) {
                route = TOPKF_ROUTE_EXACT_UNDERFILL;
                if (DUAL && T1 > T0) {
                    stream_range(x, 0, L, [&](u32x4 b, uint32_t i0) { admit4<true>(b, i0, T0, T1, A, h1); });
                    __syncthreads();
                    C = *A.cnt;
                    if (C >= k) route = TOPKF_ROUTE_BAND;
                }
            }
            certified = C >= k;
        }
    }
    uint32_t kq = k;
    if (!certified) kq = exact_route(x, L, k, outp, A, h0, h1, sm);
    count_route(p, route);
    if (*A.cnt > A.cap) count_route(p, TOPKF_ROUTE_SPILL);
    refine(A, B, h1, h0, kq, outp, k, sm);
}

template <int S, bool DUAL>
__global__ __launch_bounds__(kBlock) void persistent_kernel(Params p) {
    __shared__ Shared sm;
    const uint32_t G = gridDim.x;
    int32_t ml = *p.num_valid_rows;
    const int m_live = ml < 0 ? 0 : (ml > p.m_cap ? p.m_cap : ml);
    const int64_t slice = static_cast<int64_t>(p.n);
    const Frontier A{sm.qa, kCapA, p.ws + (2 * static_cast<int64_t>(blockIdx.x)) * slice, &sm.cnt[0]};
    const Frontier B{sm.qb, kCapB, p.ws + (2 * static_cast<int64_t>(blockIdx.x) + 1) * slice, &sm.cnt[1]};
    int row = blockIdx.x;  // first wave: one row each; then the queue
    while (row < m_live) {
        select_row<S, DUAL>(p, row, sm, A, B);
        __syncthreads();
        if (threadIdx.x == 0) sm.next_row = static_cast<int32_t>(G + atomicAdd(p.counters, 1u));
        __syncthreads();
        row = sm.next_row;
    }
    // The last workgroup to leave returns the queue and exit counters to zero.
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t done = atomicAdd(p.counters + 1, 1u);
        if (done == G - 1) {
            __threadfence();
            atomicExch(p.counters, 0u);
            atomicExch(p.counters + 1, 0u);
        }
    }
}

// KV-split mapping (Sec. 4.5, Eqs. 26-27; Sec. 5.5 "Sampled KV-split").
// Workgroups are numbered so that the parts of a row sit on one XCD (the
// dispatcher deals workgroup ids round-robin over the 8 XCDs), so the
// replicated view and the finisher's reads stay in that XCD's L2.
template <int S, bool DUAL>
__global__ __launch_bounds__(kBlock) void kvsplit_kernel(Params p) {
    __shared__ Shared sm;
    const uint32_t P = static_cast<uint32_t>(p.splits);
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t li = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const uint32_t row = li / P, part = li % P;
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    int32_t ml = *p.num_valid_rows;
    const uint32_t m_live = static_cast<uint32_t>(ml < 0 ? 0 : (ml > p.m_cap ? p.m_cap : ml));
    if (row >= m_live) return;
    const uint32_t k = p.k;
    int32_t* outp = p.out + static_cast<int64_t>(row) * k;
    const int32_t Ls = p.ke[row];
    const uint32_t L = static_cast<uint32_t>(Ls < 0 ? 0 : (Ls > p.n ? p.n : Ls));
    if (L <= k) {
        if (part == 0) {
            sentinel_row(outp, L, k);
            count_route(p, TOPKF_ROUTE_SENTINEL);
        }
        return;
    }
    const float* x = p.logits + static_cast<int64_t>(row) * p.stride;
    uint2* region = p.ws + 2 * static_cast<int64_t>(row) * p.n;  // merged candidates
    uint2* region2 = region + p.n;                                // spill / ping-pong
    uint32_t* row_count = p.counters + 64 + row;
    uint32_t* arrive = p.counters + 64 + p.m_cap + row;
    uint32_t* h0 = sm.hist[0];
    uint32_t* h1 = sm.hist[1];
    const Frontier A{sm.qa, kCapA, region, &sm.cnt[0]};
    const Frontier B{sm.qb, kCapB, region2, &sm.cnt[1]};

    bool usable = false;
    uint32_t a = 0, nv = 0, q = 0, q1 = 0;
    if constexpr (S > 0) {
        nv = view_size<S>(row, L, &a);
        q = q_primary(k, S);
        q1 = DUAL ? q_secondary(k, S) : q;
        usable = nv >= q1;
    }
    if (!usable) {
        // No usable view: part 0 runs the exact coarse route over the whole row.
        if (part != 0) return;
        const uint32_t kq = exact_route(x, L, k, outp, A, h0, h1, sm);
        count_route(p, TOPKF_ROUTE_EXACT_DIRECT);
        if (*A.cnt > A.cap) count_route(p, TOPKF_ROUTE_SPILL);
        refine(A, B, h1, h0, kq, outp, k, sm);
        return;
    }
    const uint32_t min_seg = static_cast<uint32_t>(p.min_seg);
    uint32_t Pr = ceil_div(L, min_seg);
    if (Pr > P) Pr = P;
    if (Pr < 1) Pr = 1;
    if (part >= Pr) return;
    const uint32_t chunk = ceil_div(ceil_div(L, Pr), 4) * 4;
    const uint32_t lo = part * chunk < L ? part * chunk : L;
    const uint32_t hi = lo + chunk < L ? lo + chunk : L;

    // Replicated Phase 1: every part derives the same tau0/tau1 from a_r.
    clear_hist(h0);
    clear_hist(h1);
    if (threadIdx.x == 0) { sm.cnt[0] = 0; sm.out_cnt = 0; }
    __syncthreads();
    phase1(x, a, nv, S, q, q1, h0, sm);
    const uint32_t T0 = sm.cut[0], T1 = sm.cut[1];
    // Phase 2 over this part's segment; LDS overflow goes to region2 at the
    // segment's own offset (a segment admits at most hi - lo values).
    const Frontier Aseg{sm.qa, kCapA, region2 + lo, &sm.cnt[0]};
    stream_range(x, lo, hi, [&](u32x4 b, uint32_t i0) { admit4<false>(b, i0, 0u, T0, Aseg, h1); });
    __syncthreads();
    const uint32_t nseg = sm.cnt[0];
    if (threadIdx.x == 0) sm.res[0] = atomicAdd(row_count, nseg);
    __syncthreads();
    const uint32_t base = sm.res[0];
    for (uint32_t e = threadIdx.x; e < nseg; e += kBlock) region[base + e] = fget(Aseg, e);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) sm.flag = atomicAdd(arrive, 1u) == Pr - 1 ? 1u : 0u;
    __syncthreads();
    if (!sm.flag) return;

    // Finisher: the last part to arrive sees every published candidate.
    __threadfence();
    uint32_t C = __hip_atomic_load(row_count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_store(row_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.cnt[0] = C;
        sm.out_cnt = 0;
    }
    // The merged candidates live only in `region` (a frontier with no LDS part).
    const Frontier G0{sm.qa, 0, region, &sm.cnt[0]};
    int route = TOPKF_ROUTE_PRIMARY;
    if (C < k) {
        route = TOPKF_ROUTE_EXACT_UNDERFILL;
        if (DUAL && T1 > T0) {
            __syncthreads();
            stream_range(x, 0, L, [&](u32x4 b, uint32_t i0) { admit4<true>(b, i0, T0, T1, G0, h1); });
            __syncthreads();
            C = sm.cnt[0];
            if (C >= k) route = TOPKF_ROUTE_BAND;
        }
    }
    if (C >= k) {
        // Leading-digit histogram of the merged frontier (Eq. 27).
        clear_hist(h1);
        __syncthreads();
        for (uint32_t e = threadIdx.x; e < C; e += kBlock) lds_inc(h1, region[e].y >> 21);
        __syncthreads();
        count_route(p, route);
        refine(G0, B, h1, h0, k, outp, k, sm);
    } else {
        __syncthreads();
        const uint32_t kq = exact_route(x, L, k, outp, A, h0, h1, sm);
        count_route(p, route);
        if (*A.cnt > A.cap) count_route(p, TOPKF_ROUTE_SPILL);
        refine(A, B, h1, h0, kq, outp, k, sm);
    }
}

__global__ void coarse_keys_kernel(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        out[i] = static_cast<uint16_t>(coarse_of_bits(__float_as_uint(x[i])));
}

// ------------------------------------------------------------------ host

constexpr int64_t kCounterHead = 64;  // u32 slots: [0] queue, [1] exit, rest reserved

struct DeviceInfo {
    int cus = 0;
    int occupancy = 0;  // resident 512-thread workgroups per CU
};

std::mutex g_mu;
DeviceInfo g_info[64];

topkf_status device_info(DeviceInfo* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TOPKF_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_info[dev].cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            return TOPKF_EHIP;
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, persistent_kernel<128, true>, kBlock,
                                                         0) != hipSuccess ||
            occ <= 0)
            occ = 1;
        g_info[dev].cus = cus;
        g_info[dev].occupancy = occ;
    }
    *out = g_info[dev];
    return TOPKF_OK;
}

bool plan_valid(const topkf_plan& pl) {
    if (pl.family != TOPKF_FAMILY_PERSISTENT && pl.family != TOPKF_FAMILY_KVSPLIT) return false;
    if (pl.stride != 0 && pl.stride != 64 && pl.stride != 128) return false;
    if (pl.dual != 0 && pl.dual != 1) return false;
    if (pl.family == TOPKF_FAMILY_PERSISTENT && pl.workers < 1) return false;
    if (pl.family == TOPKF_FAMILY_KVSPLIT && (pl.splits < 1 || pl.splits > 4096)) return false;
    if (pl.family == TOPKF_FAMILY_KVSPLIT && pl.min_segment < 4) return false;
    return true;
}

topkf_status make_plan(int64_t m_cap, int64_t n, int32_t cus, int32_t occupancy,
                       topkf_plan* pl) {
    if (m_cap < 0 || n < 1 || cus < 1 || !pl) return TOPKF_EINVAL;
    if (occupancy < 1) occupancy = 1;
    topkf_plan r{};
    // View policy (Sec. 5.5: s = 64 and s = 128 compile-time policies;
    // Sec. 6.4: sampling pays off for wide rows, exact localization for short).
    if (n < 16384) r.stride = 0;
    else if (n < 65536) r.stride = 64;
    else r.stride = 128;
    r.dual = r.stride ? 1 : 0;
    r.min_segment = 8192;
    const int64_t pool = static_cast<int64_t>(cus) * occupancy;
    if (r.stride == 0 || m_cap >= pool) {
        r.family = TOPKF_FAMILY_PERSISTENT;
        r.workers = static_cast<int32_t>(m_cap < pool ? (m_cap > 0 ? m_cap : 1) : pool);
        r.splits = 1;
    } else {
        r.family = TOPKF_FAMILY_KVSPLIT;
        int64_t P = (pool + m_cap - 1) / (m_cap > 0 ? m_cap : 1);
        int64_t pmax = (n + r.min_segment - 1) / r.min_segment;
        if (P > pmax) P = pmax;
        if (P < 1) P = 1;
        r.splits = static_cast<int32_t>(P);
        r.workers = 1;
    }
    *pl = r;
    return TOPKF_OK;
}

void plan_sizes(const topkf_plan& pl, int64_t m_cap, int64_t n, size_t* cb, size_t* wb) {
    *cb = static_cast<size_t>(kCounterHead + 2 * m_cap) * sizeof(uint32_t);
    const int64_t owners = pl.family == TOPKF_FAMILY_PERSISTENT ? pl.workers : m_cap;
    *wb = static_cast<size_t>(owners) * 2 * static_cast<size_t>(n) * sizeof(uint2);
}

template <int S, bool D>
hipError_t launch_family(const topkf_plan& pl, const Params& prm, hipStream_t st) {
    if (pl.family == TOPKF_FAMILY_PERSISTENT) {
        hipLaunchKernelGGL((persistent_kernel<S, D>), dim3(pl.workers), dim3(kBlock), 0, st, prm);
    } else {
        const int64_t total = static_cast<int64_t>(prm.m_cap) * pl.splits;
        const int64_t per_xcd = (total + 7) / 8;
        hipLaunchKernelGGL((kvsplit_kernel<S, D>), dim3(static_cast<uint32_t>(per_xcd * 8)),
                           dim3(kBlock), 0, st, prm);
    }
    return hipGetLastError();
}

topkf_status run(const float* logits, int64_t m_cap, int64_t n, int64_t stride,
                 const int32_t* ke, int32_t* out, const int32_t* nvr, int32_t top_k,
                 void* counters, size_t counter_bytes, void* workspace, size_t workspace_bytes,
                 const topkf_plan* override_plan, uint32_t* stats, hipStream_t st) {
    if (m_cap < 0 || n < 1 || stride < n || top_k < 1 || top_k > TOPKF_K_MAX)
        return TOPKF_EINVAL;
    if (n > 0x7FFFFFFF || m_cap > 0x7FFFFFFF) return TOPKF_EUNSUPPORTED;
    if (m_cap == 0) return TOPKF_OK;
    if (!logits || !ke || !out || !nvr || !counters) return TOPKF_EINVAL;
    topkf_plan pl;
    if (override_plan) {
        pl = *override_plan;
        if (!plan_valid(pl)) return TOPKF_EINVAL;
    } else {
        DeviceInfo di;
        const topkf_status s = device_info(&di);
        if (s != TOPKF_OK) return s;
        make_plan(m_cap, n, di.cus, di.occupancy, &pl);
    }
    size_t cb = 0, wb = 0;
    plan_sizes(pl, m_cap, n, &cb, &wb);
    if (counter_bytes < cb || workspace_bytes < wb) return TOPKF_EWORKSPACE;
    if (wb > 0 && !workspace) return TOPKF_EINVAL;
    Params prm;
    prm.logits = logits;
    prm.stride = stride;
    prm.ke = ke;
    prm.out = out;
    prm.num_valid_rows = nvr;
    prm.counters = static_cast<uint32_t*>(counters);
    prm.ws = static_cast<uint2*>(workspace);
    prm.stats = stats;
    prm.m_cap = static_cast<int32_t>(m_cap);
    prm.n = static_cast<int32_t>(n);
    prm.k = top_k;
    prm.splits = pl.splits;
    prm.min_seg = pl.min_segment;
    hipError_t e;
    switch (pl.stride * 2 + pl.dual) {
        case 0: case 1: e = launch_family<0, false>(pl, prm, st); break;
        case 128: e = launch_family<64, false>(pl, prm, st); break;
        case 129: e = launch_family<64, true>(pl, prm, st); break;
        case 256: e = launch_family<128, false>(pl, prm, st); break;
        default: e = launch_family<128, true>(pl, prm, st); break;
    }
    return e == hipSuccess ? TOPKF_OK : TOPKF_EHIP;
}

}  // namespace

extern "C" {

topkf_status topk_filtered_workspace_size(int64_t num_rows, int64_t max_kv_len,
                                          size_t* counter_bytes, size_t* workspace_bytes) {
    if (num_rows < 0 || max_kv_len < 1 || !counter_bytes || !workspace_bytes) return TOPKF_EINVAL;
    DeviceInfo di;
    const topkf_status s = device_info(&di);
    if (s != TOPKF_OK) return s;
    topkf_plan pl;
    make_plan(num_rows, max_kv_len, di.cus, di.occupancy, &pl);
    plan_sizes(pl, num_rows, max_kv_len, counter_bytes, workspace_bytes);
    return TOPKF_OK;
}

topkf_status topk_filtered(const float* logits, int64_t num_rows, int64_t max_kv_len,
                           int64_t row_stride, const int32_t* ke, int32_t* out,
                           const int32_t* num_valid_rows, int32_t top_k, void* counters,
                           size_t counter_bytes, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    return run(logits, num_rows, max_kv_len, row_stride, ke, out, num_valid_rows, top_k, counters,
               counter_bytes, workspace, workspace_bytes, nullptr, nullptr, stream);
}

topkf_status topk_filtered_debug(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                 int64_t row_stride, const int32_t* ke, int32_t* out,
                                 const int32_t* num_valid_rows, int32_t top_k, void* counters,
                                 size_t counter_bytes, void* workspace, size_t workspace_bytes,
                                 const topkf_plan* plan, uint32_t* route_stats,
                                 hipStream_t stream) {
    return run(logits, num_rows, max_kv_len, row_stride, ke, out, num_valid_rows, top_k, counters,
               counter_bytes, workspace, workspace_bytes, plan, route_stats, stream);
}

const char* topkf_status_string(topkf_status s) {
    switch (s) {
        case TOPKF_OK: return "ok";
        case TOPKF_EINVAL: return "invalid argument";
        case TOPKF_EUNSUPPORTED: return "unsupported shape";
        case TOPKF_EWORKSPACE: return "counter or workspace buffer too small";
        case TOPKF_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

topkf_status topkf_plan_for(int64_t num_rows, int64_t max_kv_len, int32_t cu_count,
                            topkf_plan* plan) {
    // The host planner assumes the occupancy of the built kernels: two
    // 512-thread workgroups per compute unit.
    return make_plan(num_rows, max_kv_len, cu_count, 2, plan);
}

topkf_status topkf_plan_workspace_size(const topkf_plan* plan, int64_t num_rows,
                                       int64_t max_kv_len, size_t* counter_bytes,
                                       size_t* workspace_bytes) {
    if (!plan || num_rows < 0 || max_kv_len < 1 || !counter_bytes || !workspace_bytes)
        return TOPKF_EINVAL;
    if (!plan_valid(*plan)) return TOPKF_EINVAL;
    plan_sizes(*plan, num_rows, max_kv_len, counter_bytes, workspace_bytes);
    return TOPKF_OK;
}

topkf_status topkf_coarse_keys(const float* x, int64_t n, uint16_t* out, hipStream_t stream) {
    if (n < 0) return TOPKF_EINVAL;
    if (n == 0) return TOPKF_OK;
    if (!x || !out) return TOPKF_EINVAL;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(coarse_keys_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, x, n, out);
    return hipGetLastError() == hipSuccess ? TOPKF_OK : TOPKF_EHIP;
}

}  // extern "C"
