// Exact FP32 row-wise Top-K for MI355X (gfx950): a sample-guided exact
// selector after "Sample-Guided Exact Top-K Selection for Long-Context Sparse
// Attention" (Secs. 4-5), behind the C ABI declared in include/topkf.h.
//
// One 512-thread workgroup (8 wave64) works on a row (or a row segment):
//   Phase 1 (Sec. 4.2, Eqs. 11-15; Sec. 5.2): the regular view
//     V = {i < L : i = a_r mod s} is projected to the 11-bit coarse key and
//     histogrammed in LDS; the first bins whose prefix reaches
//     q = ceil(K~/s) and q1 = ceil(K~1/s) give tau0 and tau1 (the plan sets
//     K~ and K~1 in quarters of K), converted once to inclusive FP32 cutoffs
//     expressed as descending integer keys.  The row's first loads are
//     already in flight while the view is histogrammed.
//   Phase 2 (Sec. 4.3, Eqs. 16-17; Sec. 5.3): one streaming pass over the
//     row with 128-bit nontemporal loads admits key <= T0 and appends the
//     (index, key) pair to the frontier.  Underfill (C < K) adds the band
//     T0 < key <= T1 (Eqs. 18-19); continued underfill, an unusable view or
//     the no-view policy take the exact coarse route (Eq. 20).
//   Phase 3 (Sec. 4.4, Eqs. 22-25; Sec. 5.4): radix refinement of the FP32
//     descending key over the frontier only, from registers (a digit window
//     of at most 11 bits over the frontier's key range, at most three rounds)
//     or, for frontiers beyond registers, 11+11+10-bit digits through two
//     ping-pong buffers of (index, key) pairs (LDS first, then a global
//     spill slice).
// Two mappings (Sec. 4.5, Sec. 5.5): a persistent pool whose workgroups take
// rows from a device queue, and a KV-split mapping in which P workgroups scan
// disjoint segments of one row (kvsplit_scan_kernel) and a second kernel on
// the same stream merges their counts and candidates and finishes each row
// (kvsplit_finish_kernel): the kernel boundary makes every part's writes
// visible without a per-workgroup cache write-back.
//
// Every wave of a workgroup runs the same trip counts, so the ballots below
// always see all 64 lanes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "topkf.h"

namespace {

constexpr int kBlock = 512;
constexpr int kWaves = kBlock / 64;
constexpr int kBins = 2048;
constexpr int kFront = 7168;                 // LDS frontier, (index, key) pairs
constexpr int kWaveCap = kFront / kWaves;    // wave-private share of it (896)
constexpr int kWaveRegs = kWaveCap / 64;     // its entries per lane (14)
constexpr int kRegs = 16;                    // contiguous frontier held in registers
constexpr int kCapA = 4096;                  // general path: LDS part of Q1 / Q2
constexpr int kRowVec = 4;      // exact route and band pass: 128-bit loads per thread per chunk
constexpr int kScanVec = 6;     // persistent sampled scan: 128-bit loads per thread in flight
constexpr int kSegVec = 8;      // KV-split scan: 128-bit loads per thread per chunk
constexpr int kSampleVec = 8;   // view samples per thread per batch
constexpr int kMaxSplits = 256; // KV-split parts per row
// Counter buffer: kCounterHead u32 slots ([0] the persistent queue), two
// slot counters per row (cooperative exact route), then for KV-split plans
// without a view one 2048-bin coarse histogram per row.
constexpr int kCounterHead = 64;
// A NaN pattern whose descending key is 0xFFFFFFFF: larger than every cutoff,
// so it marks lanes that hold no element.
constexpr uint32_t kNoElem = 0xFFFFFFFFu;
constexpr uint32_t kKeyFirst = 0x007FFFFFu;  // descending key of +inf
constexpr uint32_t kKeyLast = 0xFF800000u;   // descending key of -inf

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
    int32_t band_q;  // secondary target K~1 = ceil(band_q * K / 4)
    int32_t prim_q;  // primary target K~ = ceil(prim_q * K / 4)
    const float* hint;  // per-row proposed cutoffs (NaN: none), or null
};

// A row's caller-supplied proposal (a cutoff carried over from the previous
// decode step, as in the GVR page): when it is not NaN, its descending key
// replaces the view's cutoff.
__device__ __forceinline__ bool row_hint(const Params& p, uint32_t row, uint32_t* key) {
    const uint32_t b = __float_as_uint(p.hint[row]);
    *key = b ^ ((~static_cast<uint32_t>(static_cast<int32_t>(b) >> 31)) >> 1);
    return (b & 0x7FFFFFFFu) <= 0x7F800000u;
}

// The scalars come first so that their LDS addresses fit the 16-bit
// immediate offset of LDS instructions (no address registers needed).
struct alignas(16) Shared {
    uint32_t offs[2][kMaxSplits + 1];  // KV-split finisher: per-part prefix offsets
    alignas(16) uint32_t wsum[3][kWaves];  // per-wave totals: [0] block_find, [1], [2] scans
    uint32_t wcnt[kWaves];             // wave-private frontier sizes
    uint32_t res[4];
    uint32_t rcnt[2];                  // block_find: the count of each target's bin
    alignas(16) uint32_t wext[2][kWaves];  // per-wave smallest and largest key
    uint32_t cnt[2];
    uint32_t out_cnt;
    uint32_t tie_cnt;
    uint32_t cut[2];
    int32_t next_row;
    uint32_t part_max;  // KV-split finisher: the largest candidate count of one part
    uint32_t kext[2];  // smallest and largest key of a large frontier
    uint32_t fkey[2];  // KV-split scan: the part's flood key per kind (kNoElem: none yet)
    uint32_t fcnt[2];  // KV-split scan: copies of it in bulk batches so far
    alignas(16) uint32_t hist[2][kBins];
    uint2 front[kFront];
};
static_assert(sizeof(Shared) <= 80 * 1024, "two workgroups per CU must fit in LDS");

// Workspace geometry: every owner (a persistent worker, or a row under
// KV-split) has two slices of slice_len(n) pairs; a wave-private frontier
// spills into the first slice at wave_spill_len(n) pairs per wave.
__host__ __device__ __forceinline__ int64_t wave_spill_len(int64_t n) { return (n + 7) / 8 + 8; }
__host__ __device__ __forceinline__ int64_t slice_len(int64_t n) { return n + 128; }

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

// The inclusive FP32 cutoff of every coarse bin, computed at compile time
// (Sec. 4.3: the largest non-NaN descending key whose value still has
// c <= tau; c is monotone in the key, so {c(x) <= tau} == {key(x) <= T(tau)}).
// fp16_rne_bits is IEEE round-to-nearest-even FP32 -> FP16 in integer
// arithmetic (overflow to infinity from 65520 up, FP16 subnormals kept), the
// conversion coarse_of_bits gets from the hardware; a test compares the whole
// table with the device's own search over coarse_of_bits.  T(tau) is
// kKeyFirst - 1 (admits no non-NaN value) when even +inf lies above tau.
constexpr uint32_t fp16_rne_bits(uint32_t f) {
    const uint32_t s = (f >> 16) & 0x8000u;
    const uint32_t a = f & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return s | 0x7E00u;   // NaN
    if (a >= 0x477FF000u) return s | 0x7C00u;  // 65520 and up round to infinity
    if (a >= 0x38800000u) {                    // FP16 normal range, from 2^-14
        uint32_t v = (a >> 13) - (112u << 10);  // rebias the exponent, keep 10 mantissa bits
        const uint32_t rem = a & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (v & 1u))) v += 1;
        return s | v;
    }
    const uint32_t e = a >> 23;
    if (e < 102) return s;                     // below 2^-25: zero
    const uint32_t m = (a & 0x7FFFFFu) | 0x800000u;
    const uint32_t sh = 126 - e;               // value / 2^-24 = m >> sh
    uint32_t v = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1u);
    if (rem > half || (rem == half && (v & 1u))) v += 1;
    return s | v;
}

constexpr uint32_t coarse_of_key_exact(uint32_t k) {
    const uint32_t b = k ^ ((~static_cast<uint32_t>(static_cast<int32_t>(k) >> 31)) >> 1);
    const uint32_t h = fp16_rne_bits(b);
    const uint32_t k16 = (h & 0x8000u) ? h : (h ^ 0x7FFFu);
    return k16 >> 5;
}

struct CutTable {
    uint32_t v[kBins];
};

constexpr CutTable make_cut_table() {
    CutTable t{};
    for (uint32_t tau = 0; tau < static_cast<uint32_t>(kBins); ++tau) {
        if (coarse_of_key_exact(kKeyFirst) > tau) {
            t.v[tau] = kKeyFirst - 1;
            continue;
        }
        if (coarse_of_key_exact(kKeyLast) <= tau) {
            t.v[tau] = kKeyLast;
            continue;
        }
        uint32_t lo = kKeyFirst, hi = kKeyLast;  // c(lo) <= tau < c(hi)
        while (hi - lo > 1) {
            const uint32_t mid = lo + (hi - lo) / 2;
            if (coarse_of_key_exact(mid) <= tau) lo = mid;
            else hi = mid;
        }
        t.v[tau] = lo;
    }
    return t;
}

__constant__ CutTable kCutoff = make_cut_table();

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

__device__ __forceinline__ uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// q = ceil(K~/s) with K~ = ceil(prim_q * K / 4), 1.5K for prim_q = 6
// (Sec. 4.2); q1 = ceil(K~1/s) with K~1 = ceil(band_q * K / 4), 1.75K for
// band_q = 7 (Sec. 6.4 "Conditional rescue").  Both targets are efficiency
// knobs only (Sec. 4.6, last paragraph).
__device__ __forceinline__ uint32_t q_primary(uint32_t k, int s, int prim_q) {
    return ceil_div(ceil_div(static_cast<uint32_t>(prim_q) * k, 4), s);
}
__device__ __forceinline__ uint32_t q_secondary(uint32_t k, int s, int band_q) {
    return ceil_div(ceil_div(static_cast<uint32_t>(band_q) * k, 4), s);
}

// ------------------------------------------------------------ wave helpers

__device__ __forceinline__ uint32_t lane() { return __lane_id(); }
// The wave's index in the workgroup, in a scalar register (it is the same
// for every lane of the wave).
__device__ __forceinline__ uint32_t wave() {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)));
}

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// base + the number of set bits of m below this lane.
__device__ __forceinline__ uint32_t mbcnt_from(uint64_t m, uint32_t base) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), base));
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}

// A value every lane holds alike, moved to a scalar register.
__device__ __forceinline__ uint32_t readfirst(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Instruction-issue priority of this wave against the other waves of its
// SIMD: the latency-bound phases of a row (Phase 1, the end of the scan,
// refinement) run above the streaming loop of the co-resident workgroup,
// whose waves mostly wait on memory.
__device__ __forceinline__ void wave_priority(int level) {
    if (level == 0) __builtin_amdgcn_s_setprio(0);
    else __builtin_amdgcn_s_setprio(2);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// the row broadcasts of the GFX9 family.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xA, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xC, 0xF, false));
    return x;
}

// Minimum / maximum of x over the wave (wave-uniform), by the same DPP steps.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_min(uint32_t x) {
    const uint32_t y = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(-1, static_cast<int>(x), CTRL, ROW_MASK, 0xF, false));
    return y < x ? y : x;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max(uint32_t x) {
    const uint32_t y = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK, 0xF, false));
    return y > x ? y : x;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    x = dpp_min<0x111, 0xF>(x);
    x = dpp_min<0x112, 0xF>(x);
    x = dpp_min<0x114, 0xF>(x);
    x = dpp_min<0x118, 0xF>(x);
    x = dpp_min<0x142, 0xA>(x);
    x = dpp_min<0x143, 0xC>(x);
    return readlane(x, 63);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = dpp_max<0x111, 0xF>(x);
    x = dpp_max<0x112, 0xF>(x);
    x = dpp_max<0x114, 0xF>(x);
    x = dpp_max<0x118, 0xF>(x);
    x = dpp_max<0x142, 0xA>(x);
    x = dpp_max<0x143, 0xC>(x);
    return readlane(x, 63);
}

// Folds this wave's minimum of mn and maximum of mx into LDS.
__device__ __forceinline__ void lds_extremes(uint32_t* e, uint32_t mn, uint32_t mx) {
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane() == 0) {
        __hip_atomic_fetch_min(e, mn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_max(e + 1, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// One LDS reservation for the lanes in m; returns the first reserved slot.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, uint64_t m, uint32_t n) {
    const int leader = __builtin_ctzll(m);
    uint32_t base = 0;
    if (static_cast<int>(lane()) == leader) base = atomicAdd(counter, n);
    return readlane(base, leader);
}

__device__ __forceinline__ void lds_inc(uint32_t* h, uint32_t bin) {
    __hip_atomic_fetch_add(h + bin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void lds_add(uint32_t* h, uint32_t bin, uint32_t v) {
    __hip_atomic_fetch_add(h + bin, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Histogram count for the lanes with pred (m = their ballot, nonzero); when
// they all hit one bin (constant or heavily tied rows) a single add replaces
// up to 64 LDS atomics on one address, which the LDS would serialize.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin, bool pred, uint64_t m) {
    const int leader = __builtin_ctzll(m);
    const uint32_t b0 = readlane(bin, leader);
    if (__ballot(pred && bin == b0) == m) {
        if (static_cast<int>(lane()) == leader) lds_add(h, b0, __builtin_popcountll(m));
    } else if (pred) {
        lds_inc(h, bin);
    }
}

// Histogram count for the lanes with `on`: the lanes that share the first
// such lane's bin add their number with one atomic, the others one each (a
// group of equal keys would otherwise send up to 64 atomics to one LDS
// address, which the LDS serializes).
__device__ __forceinline__ void hist_count_lead(uint32_t* h, uint32_t bin, bool on) {
    const uint64_t m = __ballot(on);
    if (m == 0) return;
    const int leader = __builtin_ctzll(m);
    const uint32_t b0 = readlane(bin, leader);
    const bool same = on && bin == b0;
    const uint64_t me = __ballot(same);
    if (static_cast<int>(lane()) == leader) lds_add(h, b0, __builtin_popcountll(me));
    else if (on && !same) lds_inc(h, bin);
}

__device__ __forceinline__ u32x2 nt_load2(const uint2* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

__device__ __forceinline__ void nt_store2(uint2* p, uint32_t a, uint32_t b) {
    __builtin_nontemporal_store(u32x2{a, b}, reinterpret_cast<u32x2*>(p));
}

// ---------------------------------------------------------------- frontier

// Entries [0, cap) live in LDS, entries [cap, count) in a global slice.
struct Frontier {
    uint2* lds;
    uint32_t cap;
    uint2* gbl;
    uint32_t* cnt;  // LDS counter
};

__device__ __forceinline__ void fput(const Frontier& f, uint32_t slot, uint32_t idx, uint32_t key) {
    if (slot < f.cap) f.lds[slot] = make_uint2(idx, key);
    else nt_store2(f.gbl + (slot - f.cap), idx, key);
}

// Lanes with p[u] take consecutive output slots (one reservation per wave).
__device__ __forceinline__ void commit4(const bool (&p)[4], const uint32_t (&idx)[4],
                                        int32_t* outp, uint32_t k, Shared& sm) {
    uint64_t m[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) m[u] = __ballot(p[u]);
    const uint64_t any = m[0] | m[1] | m[2] | m[3];
    if (any == 0) return;
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) { c[u] = __builtin_popcountll(m[u]); tot += c[u]; }
    uint32_t base = wave_reserve(&sm.out_cnt, any, tot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (p[u]) {
            const uint32_t slot = base + mbcnt(m[u]);
            if (slot < k) outp[slot] = static_cast<int32_t>(idx[u]);
        }
        base += c[u];
    }
}

// Lanes with p[u] append (idx, key) to frontier f and count bin[u] in h.
__device__ __forceinline__ void append4(const bool (&p)[4], const uint32_t (&idx)[4],
                                        const uint32_t (&key)[4], const uint32_t (&bin)[4],
                                        const Frontier& f, uint32_t* h) {
    uint64_t m[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) m[u] = __ballot(p[u]);
    const uint64_t any = m[0] | m[1] | m[2] | m[3];
    if (any == 0) return;
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) { c[u] = __builtin_popcountll(m[u]); tot += c[u]; }
    uint32_t base = wave_reserve(f.cnt, any, tot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (m[u]) {
            if (p[u]) fput(f, base + mbcnt(m[u]), idx[u], key[u]);
            hist_add(h, bin[u], p[u], m[u]);
        }
        base += c[u];
    }
}

// Visits the frontier four entries per thread at a time: g(item[4], valid[4]).
template <class G>
__device__ __forceinline__ void for_each4(const Frontier& f, uint32_t n, G&& g) {
    const uint32_t tid = threadIdx.x;
    const uint32_t nl = n < f.cap ? n : f.cap;
    for (uint32_t e0 = 0; e0 < nl; e0 += 4 * kBlock) {
        uint2 it[4];
        bool v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t e = e0 + u * kBlock + tid;
            v[u] = e < nl;
            it[u] = v[u] ? f.lds[e] : make_uint2(0u, kNoElem);
        }
        g(it, v);
    }
    for (uint32_t e0 = nl; e0 < n; e0 += 4 * kBlock) {
        uint2 it[4];
        bool v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t e = e0 + u * kBlock + tid;
            v[u] = e < n;
            if (v[u]) {
                const u32x2 t = nt_load2(f.gbl + (e - f.cap));
                it[u] = make_uint2(t.x, t.y);
            } else {
                it[u] = make_uint2(0u, kNoElem);
            }
        }
        g(it, v);
    }
}

__device__ __forceinline__ uint2 fget(const Frontier& f, uint32_t e) {
    if (e < f.cap) return f.lds[e];
    const u32x2 t = nt_load2(f.gbl + (e - f.cap));
    return make_uint2(t.x, t.y);
}

// Wave-private frontier: wave w appends into its own share
// front[w * kWaveCap, (w + 1) * kWaveCap) of the LDS frontier and then into its
// own global spill range.  The running size is wave-uniform (it only changes
// by popcounts of ballots), so placing an entry needs no atomic.
struct WaveFrontier {
    uint2* lds;
    uint2* gbl;
    uint32_t n;
};

__device__ __forceinline__ void wput(const WaveFrontier& f, uint32_t slot, uint32_t idx,
                                     uint32_t key) {
    if (slot < kWaveCap) f.lds[slot] = make_uint2(idx, key);
    else nt_store2(f.gbl + (slot - kWaveCap), idx, key);
}

// Wave-private frontier entries are (index, FP32 bit pattern) pairs; the
// descending key is formed when they are read back (desc_key).

// Lanes with p[u] append (idx[u], bits[u]) to the wave frontier.  The running
// count is wave-uniform, so each slot is that count plus the lane's rank
// among the lanes that append.
__device__ __forceinline__ void wappend4(const bool (&p)[4], const uint32_t (&idx)[4],
                                         const uint32_t (&bits)[4], WaveFrontier& f) {
    uint64_t m[4];
    uint32_t c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        m[u] = __ballot(p[u]);
        c[u] = __builtin_popcountll(m[u]);
    }
    if ((m[0] | m[1] | m[2] | m[3]) == 0) return;
    uint32_t n = f.n;
    const uint32_t end = n + c[0] + c[1] + c[2] + c[3];
    if (end <= static_cast<uint32_t>(kWaveCap)) {  // wave-uniform: every new slot is in LDS
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint2* at = f.lds + n;
            if (p[u]) at[mbcnt(m[u])] = make_uint2(idx[u], bits[u]);
            n += c[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (p[u]) wput(f, n + mbcnt(m[u]), idx[u], bits[u]);
            n += c[u];
        }
    }
    f.n = end;
}

// ------------------------------------------------------------ block scans

// The sum of the per-wave totals of the waves below this one, and (*all) of
// all eight, from one broadcast read of the eight totals.
__device__ __forceinline__ uint32_t waves_below(const uint32_t* wt, uint32_t* all) {
    const uint4 a = reinterpret_cast<const uint4*>(wt)[0];
    const uint4 b = reinterpret_cast<const uint4*>(wt)[1];
    const uint32_t w = wave();
    uint32_t s = 0;
    s += w > 0 ? a.x : 0u;
    s += w > 1 ? a.y : 0u;
    s += w > 2 ? a.z : 0u;
    s += w > 3 ? a.w : 0u;
    s += w > 4 ? b.x : 0u;
    s += w > 5 ? b.y : 0u;
    s += w > 6 ? b.z : 0u;
    *all = a.x + a.y + a.z + a.w + b.x + b.y + b.z + b.w;
    return s;
}

__device__ __forceinline__ void clear_hist(uint32_t* h) {
    reinterpret_cast<uint4*>(h)[threadIdx.x] = make_uint4(0, 0, 0, 0);
}

// For each target t[i] (1 <= t[i] <= sum of hist), finds b = min{b : H(b) >=
// t[i]} and H(b - 1) (Eqs. 15, 23), written to sm.res[2i], sm.res[2i + 1],
// and the count of bin b, written to sm.rcnt[i].
// Each thread owns 4 consecutive bins.  Reads hist before its first barrier
// and ends with a barrier, so hist may be rewritten right after it returns.
template <int NT>
__device__ __forceinline__ void block_find(const uint32_t* hist, const uint32_t (&t)[NT], Shared& sm) {
    const uint32_t tid = threadIdx.x;
    // Defaults keep every later LDS index in range should a target exceed
    // the histogram total (only possible for NaN inputs, which the contract
    // excludes); the finding thread overwrites them after the first barrier.
    if (tid == 0) {
#pragma unroll
        for (int i = 0; i < NT; ++i) { sm.res[2 * i] = kBins - 1; sm.res[2 * i + 1] = 0; sm.rcnt[i] = 0; }
    }
    const uint4 v = reinterpret_cast<const uint4*>(hist)[tid];
    const uint32_t s = v.x + v.y + v.z + v.w;
    const uint32_t incl = wave_incl_scan(s);
    if (lane() == 63) sm.wsum[0][wave()] = incl;
    __syncthreads();
    uint32_t all;
    const uint32_t excl = waves_below(sm.wsum[0], &all) + incl - s;
    // The bin within the thread's four: the number of partial sums below
    // the target, with no branch and no per-bin constant (such constants get
    // spilled, and the reload's wait would also wait for every load the
    // thread has in flight).
    const uint32_t a1 = excl + v.x, a2 = a1 + v.y, a3 = a2 + v.z;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (excl < t[i] && t[i] <= excl + s) {
            const uint32_t st = (a1 < t[i] ? 1u : 0u) + (a2 < t[i] ? 1u : 0u) + (a3 < t[i] ? 1u : 0u);
            const uint32_t acc = st == 0 ? excl : st == 1 ? a1 : st == 2 ? a2 : a3;
            const uint32_t c = st == 0 ? v.x : st == 1 ? v.y : st == 2 ? v.z : v.w;
            sm.res[2 * i] = 4 * tid + st;
            sm.res[2 * i + 1] = acc;
            sm.rcnt[i] = c;
        }
    }
    __syncthreads();
}

// Exclusive prefix of one value per thread over the block; *total gets the
// sum.  Uses per-wave total slot `slot` (1 or 2) and one barrier: the next
// scan on the same slot must be separated from this one by another barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, Shared& sm,
                                                    int slot) {
    const uint32_t incl = wave_incl_scan(v);
    if (lane() == 63) sm.wsum[slot][wave()] = incl;
    __syncthreads();
    return waves_below(sm.wsum[slot], total) + incl - v;
}

// Sec. 4.3: the inclusive FP32 cutoff of coarse bin tau, as the largest
// non-NaN descending key whose value still has c <= tau, searched on the
// device with the hardware conversion (the check of the compile-time table).  c is monotone in the
// key, so {c(x) <= tau} == {key(x) <= cutoff(tau)}.  A 64-way search by one
// whole wave: each round splits the interval over the lanes.  Returns
// kKeyFirst - 1 (admits no non-NaN value) when even +inf lies above tau.
__device__ __forceinline__ uint32_t wave_cutoff(uint32_t tau) {
    if (coarse_of_bits(bits_of_key(kKeyFirst)) > tau) return kKeyFirst - 1;
    if (coarse_of_bits(bits_of_key(kKeyLast)) <= tau) return kKeyLast;
    uint32_t lo = kKeyFirst, hi = kKeyLast;  // c(lo) <= tau < c(hi)
    while (hi - lo > 1) {
        const uint32_t step = (hi - lo + 63) / 64;
        const uint32_t probe = lo + (lane() + 1) * step;
        const bool ok = probe < hi && coarse_of_bits(bits_of_key(probe)) <= tau;
        const uint32_t nt = __builtin_popcountll(__ballot(ok));
        if (nt < 64) {
            const uint32_t nhi = lo + (nt + 1) * step;  // the first failing probe
            if (nhi < hi) hi = nhi;
        }
        lo += nt * step;
    }
    return lo;
}

// ------------------------------------------------------------- streaming

// [lo, hi) of row x split for 128-bit loads: an unaligned head of up to 3
// elements, a 16-byte aligned body of nvec vectors, a tail of up to 3.
struct Span {
    const float* x;
    uint32_t lo, hi, head, vlo, nvec, tlo, nscal;
};

__device__ __forceinline__ Span make_span(const float* x, uint32_t lo, uint32_t hi) {
    Span s;
    s.x = x;
    s.lo = lo;
    s.hi = hi > lo ? hi : lo;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(x + lo);
    uint32_t head = static_cast<uint32_t>(((16u - (addr & 15u)) & 15u) >> 2);
    if (head > s.hi - lo) head = s.hi - lo;
    s.head = head;
    s.vlo = lo + head;
    s.nvec = (s.hi - s.vlo) >> 2;
    s.tlo = s.vlo + 4 * s.nvec;
    s.nscal = head + (s.hi - s.tlo);
    return s;
}

// Body vector vi of a span, or the filler kNoElem when vi is past its end.
__device__ __forceinline__ u32x4 in_span(const u32x4& v, uint32_t vi, uint32_t nvec) {
    return vi < nvec ? v : u32x4{kNoElem, kNoElem, kNoElem, kNoElem};
}

// Loads this thread's vectors base + u * kBlock + tid (u < U) of the span
// body.  In a partial chunk, lanes past the end load the body's last vector
// instead (every load in bounds and unconditional, so that the loads issue
// back to back: a filler written into a load's destination first makes the
// compiler wait on earlier loads); consumers apply in_span.  nvec >= 1.
template <int U>
__device__ __forceinline__ void load_chunk(const Span& sp, uint32_t base, u32x4 (&v)[U]) {
    const u32x4* xb = reinterpret_cast<const u32x4*>(sp.x + sp.vlo);
    if (base + U * kBlock <= sp.nvec) {  // a whole chunk inside the span: no per-lane bounds
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(xb + base + u * kBlock + threadIdx.x);
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t vi = base + u * kBlock + threadIdx.x;
        v[u] = __builtin_nontemporal_load(xb + (vi < sp.nvec ? vi : sp.nvec - 1));
    }
}

// The chunked part of a span scan: `a` holds the first chunk (loads issued);
// later chunks are double buffered in two register sets used in turn (no
// copies between them), the next chunk in flight while the current one is
// processed; mid() runs as the last chunk is taken up.
template <int U, class F, class Mid>
__device__ __forceinline__ void chunk_loop(const Span& sp, u32x4 (&a)[U], F&& f, Mid&& mid) {
    const uint32_t tid = threadIdx.x;
    constexpr uint32_t C = kBlock * U;
    if (sp.nvec == 0) {
        mid();
        return;
    }
    u32x4 b[U];
    uint32_t base = 0;
    while (true) {
        // a holds the chunk at base
        bool more = base + C < sp.nvec;
        if (more) load_chunk<U>(sp, base + C, b);
        else mid();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t vi = base + u * kBlock + tid;
            f(in_span(a[u], vi, sp.nvec), sp.vlo + 4 * vi);
        }
        if (!more) break;
        base += C;
        // b holds the chunk at base
        more = base + C < sp.nvec;
        if (more) load_chunk<U>(sp, base + C, a);
        else mid();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t vi = base + u * kBlock + tid;
            f(in_span(b[u], vi, sp.nvec), sp.vlo + 4 * vi);
        }
        if (!more) break;
        base += C;
    }
}

// Calls f(bits4, index of bits4.x) over every element of the span.  issue()
// runs first (loads whose results pre() needs, ahead of the chunk in the
// in-order load queue), then the first chunk (U vectors per thread) and the
// head/tail elements are loaded, then pre() runs, so their latency overlaps
// pre().  Later chunks are double buffered in two register sets used in turn
// (no copies between them): the next chunk is in flight while the current
// one is processed.  mid() runs exactly once, as the last chunk is taken up
// (after that chunk's loads were issued), or after the head/tail elements
// when there is no chunk.  Every thread of the block must call it with the
// same span.
template <int U, class Issue, class Pre, class F, class Mid>
__device__ __forceinline__ void scan_span(const Span& sp, Issue&& issue, Pre&& pre, F&& f, Mid&& mid) {
    const uint32_t tid = threadIdx.x;
    issue();
    u32x4 a[U];
    if (sp.nvec) load_chunk<U>(sp, 0, a);
    const uint32_t se = tid < sp.head ? sp.lo + tid : sp.tlo + (tid - sp.head);
    uint32_t sb = kNoElem;
    if (tid < sp.nscal) sb = __float_as_uint(sp.x[se]);
    pre();
    if (sp.nscal) f(u32x4{sb, kNoElem, kNoElem, kNoElem}, se);
    chunk_loop<U>(sp, a, f, mid);
}

// scan_span with the element step chosen after pre(): sel() returns 0, 1 or
// 2 and the body is scanned with f0, f1 or f2 (one chunk loop compiled per
// step, so a scan runs only the code of its own step).  Only the last N
// steps are compiled (N = 2: sel() never returns 0; N = 1: always f1).
template <int U, int N, class Issue, class Pre, class Sel, class F0, class F1, class F2, class Mid>
__device__ __forceinline__ void scan_span_sel(const Span& sp, Issue&& issue, Pre&& pre, Sel&& sel,
                                              F0&& f0, F1&& f1, F2&& f2, Mid&& mid) {
    const uint32_t tid = threadIdx.x;
    issue();
    u32x4 a[U];
    if (sp.nvec) load_chunk<U>(sp, 0, a);
    const uint32_t se = tid < sp.head ? sp.lo + tid : sp.tlo + (tid - sp.head);
    uint32_t sb = kNoElem;
    if (tid < sp.nscal) sb = __float_as_uint(sp.x[se]);
    pre();
    const int which = sel();
    const u32x4 s4{sb, kNoElem, kNoElem, kNoElem};
    if (N > 2 && which == 0) {
        if (sp.nscal) f0(s4, se);
        chunk_loop<U>(sp, a, f0, mid);
    } else if (N < 2 || which == 1) {
        if (sp.nscal) f1(s4, se);
        chunk_loop<U>(sp, a, f1, mid);
    } else {
        if (sp.nscal) f2(s4, se);
        chunk_loop<U>(sp, a, f2, mid);
    }
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{}):
// a loop whose index is a compile-time constant in every step, so that arrays
// indexed by it stay in registers however large the step is.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_from<0, N>(f);
}

// Vector j of this thread's share of a span body: body vector j * kBlock + tid
// (as load_chunk: lanes past the end load the body's last vector; consumers
// apply in_span).  nvec >= 1.
__device__ __forceinline__ void load_vec(const Span& sp, uint32_t j, u32x4& v) {
    const u32x4* xb = reinterpret_cast<const u32x4*>(sp.x + sp.vlo);
    const uint32_t vi = j * kBlock + threadIdx.x;
    v = __builtin_nontemporal_load(xb + (vi < sp.nvec ? vi : sp.nvec - 1));
}

// The body of a span as a rolling ring of V vector registers per thread: r[j]
// holds (or has in flight) this thread's vector j0 + j, and each slot is
// refilled with the vector V further on as soon as it has been processed, so
// that about V - 1 vectors per thread stay in flight at all times (double
// buffering in the same registers would let the count fall to zero at every
// switch).  The caller has issued vectors 0 .. V-1.  mid() runs once, when
// the last load has been issued.
template <int V, class F, class Mid>
__device__ __forceinline__ void ring_loop(const Span& sp, u32x4 (&r)[V], F&& f, Mid&& mid) {
    const uint32_t tid = threadIdx.x;
    const uint32_t nv = sp.nvec;
    const u32x4* xv = reinterpret_cast<const u32x4*>(sp.x + sp.vlo) + tid;
    uint32_t j0 = 0;
    // Steady state: this round's refills are whole rows of the block.
    while ((j0 + 2 * V) * kBlock <= nv) {
        static_for<V>([&](auto J) {
            constexpr int j = decltype(J)::value;
            f(r[j], sp.vlo + 4 * ((j0 + j) * kBlock + tid));
            r[j] = __builtin_nontemporal_load(xv + (j0 + j + V) * kBlock);
        });
        j0 += V;
    }
    // Last two rounds: refills (and vectors) may be partial or absent.
    static_for<V>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const uint32_t vi = (j0 + j) * kBlock + tid;
        if ((j0 + j) * kBlock < nv) f(in_span(r[j], vi, nv), sp.vlo + 4 * vi);
        if ((j0 + j + V) * kBlock < nv) load_vec(sp, j0 + j + V, r[j]);
    });
    mid();
    j0 += V;
    static_for<V>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const uint32_t vi = (j0 + j) * kBlock + tid;
        if ((j0 + j) * kBlock < nv) f(in_span(r[j], vi, nv), sp.vlo + 4 * vi);
    });
}

// scan_span over a rolling ring of V vectors per thread, with the element
// function chosen once, after pre(): fa when sel() holds, else fb (each has
// its own loop).  The first V vectors per thread and the head/tail elements
// are in flight while pre() runs.
template <int V, class Issue, class Pre, class Sel, class FA, class FB, class Mid>
__device__ __forceinline__ void scan_span2(const Span& sp, Issue&& issue, Pre&& pre, Sel&& sel,
                                           FA&& fa, FB&& fb, Mid&& mid) {
    const uint32_t tid = threadIdx.x;
    issue();
    // Nothing else is in flight here; an explicit wait lets the ring's loads
    // issue back to back (the compiler otherwise cannot tell that no earlier
    // load still targets the ring's registers, and waits between them).
    __builtin_amdgcn_s_waitcnt(0);
    u32x4 r[V];
    if (V * kBlock <= sp.nvec) {  // block-uniform: the whole ring exists
        const u32x4* xv = reinterpret_cast<const u32x4*>(sp.x + sp.vlo) + tid;
        static_for<V>([&](auto J) {
            r[decltype(J)::value] = __builtin_nontemporal_load(xv + decltype(J)::value * kBlock);
        });
    } else if (sp.nvec) {
        static_for<V>([&](auto J) {
            if (decltype(J)::value * kBlock < sp.nvec) load_vec(sp, decltype(J)::value, r[decltype(J)::value]);
        });
    }
    const uint32_t se = tid < sp.head ? sp.lo + tid : sp.tlo + (tid - sp.head);
    uint32_t sb = kNoElem;
    if (tid < sp.nscal) sb = __float_as_uint(sp.x[se]);
    pre();
    wave_priority(0);
    if (sel()) {
        if (sp.nscal) fa(u32x4{sb, kNoElem, kNoElem, kNoElem}, se);
        ring_loop<V>(sp, r, fa, mid);
    } else {
        if (sp.nscal) fb(u32x4{sb, kNoElem, kNoElem, kNoElem}, se);
        ring_loop<V>(sp, r, fb, mid);
    }
    wave_priority(1);
}

struct NoPre {
    __device__ void operator()() const {}
};

template <int U, class Pre, class F, class Mid>
__device__ __forceinline__ void scan_span(const Span& sp, Pre&& pre, F&& f, Mid&& mid) {
    scan_span<U>(sp, NoPre{}, pre, f, mid);
}

template <int U, class Pre, class F>
__device__ __forceinline__ void scan_span(const Span& sp, Pre&& pre, F&& f) {
    scan_span<U>(sp, NoPre{}, pre, f, NoPre{});
}

// Phase 2 admission of one 4-element group (Eqs. 16-17): key <= khi, and
// key > klo for the band of Eq. 18; admitted pairs go to the wave frontier.
template <bool BAND>
__device__ __forceinline__ void admit4(u32x4 b, uint32_t i0, uint32_t klo, uint32_t khi,
                                       WaveFrontier& f) {
    uint32_t idx[4], bits[4];
    bool p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t key = desc_key(b[u]);
        p[u] = key <= khi && (!BAND || key > klo);
        idx[u] = i0 + u;
        bits[u] = b[u];
    }
    wappend4(p, idx, bits, f);
}

// The same admission when the cutoff value is >= +0, with vt its bit pattern:
// a non-negative pattern compared as a signed integer orders like its value
// and every negative pattern (and the kNoElem filler) lies below, so
// (int)bits >= (int)vt is the predicate key <= T0 in one compare.
__device__ __forceinline__ void admit4_raw(u32x4 b, uint32_t i0, uint32_t vt, WaveFrontier& f) {
    uint32_t idx[4], bits[4];
    bool p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        p[u] = static_cast<int32_t>(b[u]) >= static_cast<int32_t>(vt);
        idx[u] = i0 + u;
        bits[u] = b[u];
    }
    wappend4(p, idx, bits, f);
}

// ------------------------------------------------------------ row pieces

__device__ __forceinline__ void sentinel_row(int32_t* outp, uint32_t L, uint32_t k) {
    for (uint32_t j = threadIdx.x; j < k; j += kBlock) outp[j] = j < L ? static_cast<int32_t>(j) : -1;
}

__device__ __forceinline__ void count_route(const Params& p, int route) {
    if (p.stats && threadIdx.x == 0) atomicAdd(p.stats + route, 1u);
}

// The first batch of view samples of phase1 (sample j0 + u * kBlock + tid).
__device__ __forceinline__ void view_batch(const float* x, uint32_t a, uint32_t nv, int s, uint32_t j0,
                                           uint32_t (&b)[kSampleVec]) {
#pragma unroll
    for (int u = 0; u < kSampleVec; ++u) {
        const uint32_t j = j0 + u * kBlock + threadIdx.x;
        b[u] = j < nv ? __float_as_uint(x[a + j * s]) : kNoElem;
    }
}

// The FP32 cutoffs T(tau0) and T(tau1) of Phase 1 (block-uniform).
struct Cuts {
    uint32_t t0, t1;
};

// Counts a batch of view samples (kNoElem: none) in the coarse histogram h.
__device__ __forceinline__ void view_count(const uint32_t (&b)[kSampleVec], uint32_t* h) {
#pragma unroll
    for (int u = 0; u < kSampleVec; ++u)
        if (b[u] != kNoElem) lds_inc(h, coarse_of_bits(b[u]));
}

// Phase 1: coarse histogram of the view into h (cleared and visible; `first`
// is the first batch of samples when it was loaded ahead, else samples
// [0, counted) are already in h), tau0 and tau1 (Eq. 15), and their
// inclusive FP32 cutoffs from the compile-time table.  All sample loads of a
// batch are issued before any is used.  Ends with a barrier.
__device__ __forceinline__ Cuts phase1(const float* x, uint32_t a, uint32_t nv, int s, uint32_t q, uint32_t q1,
                       uint32_t* h, Shared& sm, const uint32_t* first = nullptr,
                       uint32_t counted = 0) {
    const uint32_t tid = threadIdx.x;
    if (first) {
#pragma unroll
        for (int u = 0; u < kSampleVec; ++u)
            if (first[u] != kNoElem) lds_inc(h, coarse_of_bits(first[u]));
        counted = kBlock * kSampleVec;
    }
    for (uint32_t j0 = counted; j0 < nv; j0 += kBlock * kSampleVec) {
        uint32_t b[kSampleVec];
#pragma unroll
        for (int u = 0; u < kSampleVec; ++u) {
            const uint32_t j = j0 + u * kBlock + tid;
            b[u] = j < nv ? __float_as_uint(x[a + j * s]) : kNoElem;
        }
#pragma unroll
        for (int u = 0; u < kSampleVec; ++u)
            if (b[u] != kNoElem) lds_inc(h, coarse_of_bits(b[u]));
    }
    __syncthreads();
    const uint32_t t[2] = {q, q1};
    block_find<2>(h, t, sm);
    const uint32_t tau0 = readfirst(sm.res[0]), tau1 = readfirst(sm.res[2]);
    return Cuts{kCutoff.v[tau0], kCutoff.v[tau1]};
}

// Records each wave's frontier size and returns the total (ends with a barrier).
__device__ __forceinline__ uint32_t publish_waves(const WaveFrontier& wf, Shared& sm) {
    if (lane() == 0) sm.wcnt[wave()] = wf.n;
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += sm.wcnt[w];
    return c;
}

// Exact coarse route (Sec. 4.3, Eq. 20) over [0, L): coarse histogram of
// every value, tau* = min{b : C(b) >= K}, then one classification pass (from
// registers when the row fits one chunk, else a second read) that
// commits c < tau* to the output and retains c == tau* in the wave frontier.
// Returns k0 = K - |E0|; the committed count is left in sm.out_cnt and the
// frontier sizes in sm.wcnt.  hc: a 2048-bin LDS histogram (any contents).
template <bool REGS>
__device__ __forceinline__ uint32_t exact_route(const float* x, uint32_t L, uint32_t k,
                                                int32_t* outp, WaveFrontier& wf, uint32_t* hc,
                                                Shared& sm) {
    __syncthreads();  // earlier readers of the frontier and histograms are done
    clear_hist(hc);
    if (threadIdx.x == 0) sm.out_cnt = 0;
    wf.n = 0;
    __syncthreads();
    const Span sp = make_span(x, 0, L);
    auto count = [&](u32x4 b, uint32_t) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (b[u] != kNoElem) lds_inc(hc, coarse_of_bits(b[u]));
    };
    uint32_t tau = 0;
    auto classify = [&](u32x4 b, uint32_t i0) {
        bool com[4], ret[4];
        uint32_t idx[4], bits[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool valid = b[u] != kNoElem;
            const uint32_t cc = coarse_of_bits(b[u]);
            com[u] = valid && cc < tau;
            ret[u] = valid && cc == tau;
            idx[u] = i0 + u;
            bits[u] = b[u];
        }
        commit4(com, idx, outp, k, sm);
        wappend4(ret, idx, bits, wf);
    };
    const uint32_t t[1] = {k};
    if (REGS && sp.nvec <= static_cast<uint32_t>(kBlock * kRowVec)) {
        // A row of at most one chunk stays in registers: one read serves the
        // histogram and the classification (Sec. 5.5 "Row-local exact").
        const uint32_t tid = threadIdx.x;
        u32x4 v[kRowVec];
#pragma unroll
        for (int u = 0; u < kRowVec; ++u) v[u] = u32x4{kNoElem, kNoElem, kNoElem, kNoElem};
        if (sp.nvec) load_chunk<kRowVec>(sp, 0, v);
        const uint32_t se = tid < sp.head ? sp.lo + tid : sp.tlo + (tid - sp.head);
        const u32x4 sb{tid < sp.nscal ? __float_as_uint(sp.x[se]) : kNoElem, kNoElem, kNoElem, kNoElem};
        count(sb, se);
#pragma unroll
        for (int u = 0; u < kRowVec; ++u) v[u] = in_span(v[u], u * kBlock + tid, sp.nvec);
#pragma unroll
        for (int u = 0; u < kRowVec; ++u) count(v[u], 0u);
        __syncthreads();
        block_find<1>(hc, t, sm);
        tau = sm.res[0];
        const uint32_t before = sm.res[1];
        if (sp.nscal) classify(sb, se);
#pragma unroll
        for (int u = 0; u < kRowVec; ++u) classify(v[u], sp.vlo + 4 * (u * kBlock + tid));
        publish_waves(wf, sm);
        return k - before;
    }
    scan_span<kRowVec>(sp, NoPre{}, count);
    __syncthreads();
    block_find<1>(hc, t, sm);
    tau = sm.res[0];
    const uint32_t before = sm.res[1];
    scan_span<kRowVec>(sp, NoPre{}, classify);
    publish_waves(wf, sm);
    return k - before;
}

// Phase 3 (Sec. 4.4) with the whole frontier in registers: each thread holds
// up to R (index, key) entries given by load(u, idx, key); kq is the
// remaining quota and out_base the number of indices committed before.  A
// radix selection over the descending FP32 key whose digit window follows
// the frontier: the active keys lie in [lo, hi] (at first the frontier's
// smallest and largest key), a round's digit is (key - lo) >> sh with sh the
// smallest shift that maps [lo, hi] into the 2048 bins, b = min{b : H(b) >=
// kq} (Eq. 23), the lower bins are committed (Eq. 24) and bin b is kept with
// [lo, hi] narrowed to it (Eq. 25).  Over the whole 32-bit key range the
// rounds are the 11 + 11 + 10 digits; over the narrow range that a frontier
// of candidates spans, one round usually leaves a boundary group of a few
// entries.  A boundary group of at most 64 entries is finished by one wave
// (rank by full key); after a round with sh == 0 the boundary group holds
// equal keys and its first `need` entries fill the output.  Output slots come
// from block prefix sums and are staged in LDS (the frontier buffer is free
// once the entries are in registers), then written out with coalesced
// stores.  hA, hB: two 2048-bin LDS histograms (any contents).  Writes
// out[out_base, k).  KNOWN: the caller gives the entries' smallest and
// largest key, has cleared hA and made it visible, and reads nothing from the
// frontier buffer (it becomes the stage without a barrier).
template <int R, bool KNOWN = false, class Load>
__device__ __forceinline__ void refine_regs(Load&& load, uint32_t* hA, uint32_t* hB, uint32_t kq,
                                            uint32_t out_base, int32_t* outp, uint32_t k,
                                            Shared& sm, uint32_t lo_known = 0,
                                            uint32_t hi_known = 0) {
    // load(u, idx, key) issues its load unconditionally (a clamped address
    // for a slot without an entry) and returns whether slot u holds one, so
    // that the R loads of a thread are in flight together.
    uint32_t idx[R], key[R];
    uint32_t act = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) act |= load(u, idx[u], key[u]) ? 1u << u : 0u;
    uint32_t lo = lo_known, hi = hi_known;
    if constexpr (!KNOWN) {
        uint32_t mn = kNoElem, mx = 0;
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const bool on = (act >> u) & 1u;
            mn = on && key[u] < mn ? key[u] : mn;
            mx = on && key[u] > mx ? key[u] : mx;
        }
        mn = wave_min(mn);
        mx = wave_max(mx);
        if (lane() == 0) {
            sm.wext[0][wave()] = mn;
            sm.wext[1][wave()] = mx;
        }
        clear_hist(hA);
        __syncthreads();  // entries are in registers (the frontier buffer becomes the stage)
        const uint4* we = reinterpret_cast<const uint4*>(&sm.wext[0][0]);
        const uint4 a = we[0], b = we[1], c = we[2], d = we[3];
        lo = min(min(min(a.x, a.y), min(a.z, a.w)), min(min(b.x, b.y), min(b.z, b.w)));
        hi = max(max(max(c.x, c.y), max(c.z, c.w)), max(max(d.x, d.y), max(d.z, d.w)));
    }
    uint32_t* stage = reinterpret_cast<uint32_t*>(sm.front);
    const uint32_t base0 = out_base;
    // Each round at least halves the window's bit length in the worst case
    // (32 -> 21 -> 10 -> 0 bits beyond the digit), so the third round has
    // sh == 0 and is the last.
    for (int j = 0; j < 3; ++j) {
        const uint32_t span = hi - lo;
        const uint32_t bl = span ? 32u - static_cast<uint32_t>(__builtin_clz(span)) : 0u;
        const uint32_t sh = bl > 11 ? bl - 11 : 0u;
        {
            // A wave whose first slot has at least 8 lanes in the bin of its
            // first active lane counts with hist_count_lead (heavily tied
            // rows would otherwise send up to 64 atomics to one address per
            // slot); other waves use plain atomics.
            const uint32_t d0 = (key[0] - lo) >> sh;
            const bool a0 = act & 1u;
            const uint64_t m0 = __ballot(a0);
            bool tied = false;
            if (m0) {
                const uint32_t b0 = readlane(d0, __builtin_ctzll(m0));
                tied = __builtin_popcountll(__ballot(a0 && d0 == b0)) >= 8;
            }
            if (tied) {
#pragma unroll
                for (int u = 0; u < R; ++u) hist_count_lead(hA, (key[u] - lo) >> sh, (act >> u) & 1u);
            } else {
#pragma unroll
                for (int u = 0; u < R; ++u)
                    if ((act >> u) & 1u) lds_inc(hA, (key[u] - lo) >> sh);
            }
        }
        clear_hist(hB);  // the next round's histogram, or the boundary list
        __syncthreads();
        const uint32_t t[1] = {kq};
        block_find<1>(hA, t, sm);
        const uint32_t b = sm.res[0], before = sm.res[1], inb = sm.rcnt[0];
        const bool exact_fill = before + inb == kq;  // the boundary group fits exactly
        const bool last = exact_fill || sh == 0;
        const bool small = !last && inb <= 64;
        const uint32_t need = kq - before;
        // com: committed entries; grp: the boundary bin's entries (ties
        // filling the last slots after a last round, else kept)
        uint32_t com = 0, grp = 0;
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const uint32_t d = (key[u] - lo) >> sh;
            const bool on = (act >> u) & 1u;
            if (on && (d < b || (exact_fill && d == b))) com |= 1u << u;
            if (on && !exact_fill && d == b) grp |= 1u << u;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(
            static_cast<uint32_t>(__builtin_popcount(com)) |
                (static_cast<uint32_t>(__builtin_popcount(grp)) << 16),
            &tot, sm, 1);
        const uint32_t tot_c = tot & 0xFFFFu;
        const uint32_t pc0 = out_base + (ex & 0xFFFFu), pg0 = ex >> 16;
        // A boundary group of at most 64 entries is finished by one wave:
        // gathered into a list (in hB), each entry's rank among the group by
        // full key (equal keys by list position) is its order, and the
        // `need` first take the remaining slots: the selection the remaining
        // rounds would make.
        uint2* list = reinterpret_cast<uint2*>(hB);
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const uint32_t below = (1u << u) - 1u;
            if ((com >> u) & 1u) {
                const uint32_t pc = pc0 + static_cast<uint32_t>(__builtin_popcount(com & below));
                if (pc < k) stage[pc] = idx[u];
            }
            if ((grp >> u) & 1u) {
                const uint32_t pg = pg0 + static_cast<uint32_t>(__builtin_popcount(grp & below));
                if (last) {
                    const uint32_t slot = out_base + tot_c + pg;
                    if (pg < need && slot < k) stage[slot] = idx[u];
                } else if (small) {
                    list[pg] = make_uint2(idx[u], key[u]);
                }
            }
        }
        if (last) break;
        if (small) {
            __syncthreads();
            if (wave() == 0) {
                const uint32_t l = lane();
                const uint2 mine = l < inb ? list[l] : make_uint2(0u, kNoElem);
                uint32_t rank = 0;
                for (uint32_t e0 = 0; e0 < inb; e0 += 8) {
#pragma unroll
                    for (uint32_t jj = 0; jj < 8; ++jj) {
                        const uint32_t e = e0 + jj;
                        const uint32_t ke = readlane(mine.y, static_cast<int>(e));
                        rank += (e < inb && (ke < mine.y || (ke == mine.y && e < l))) ? 1u : 0u;
                    }
                }
                if (l < inb && rank < need) stage[out_base + tot_c + rank] = mine.x;
            }
            break;
        }
        act = grp;
        out_base += tot_c;
        kq = need;
        lo += b << sh;
        const uint64_t top = static_cast<uint64_t>(lo) + ((1ull << sh) - 1ull);
        if (top < hi) hi = static_cast<uint32_t>(top);
        uint32_t* th = hA; hA = hB; hB = th;
    }
    __syncthreads();
    for (uint32_t j = base0 + threadIdx.x; j < k; j += kBlock) outp[j] = static_cast<int32_t>(stage[j]);
}

// Phase 3 (Sec. 4.4), general form: refinement of frontier `cur` whose leading-digit
// histogram is in hc, with remaining quota kq.  Frontier counts and hc must
// be visible (barrier done).  Commits exactly kq more indices.
__device__ __forceinline__ void refine(Frontier cur, Frontier nxt, uint32_t* hc, uint32_t* hn, uint32_t kq,
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
        if (inb == n && !exact_fill) {
            // The whole frontier shares digit j (so before == 0): nothing is
            // committed or discarded in this round.
            if (j == 2) {
                // All keys are equal: any `need` entries complete the output.
                const uint32_t base = sm.out_cnt;
                for (uint32_t e = tid; e < need; e += kBlock)
                    if (base + e < k) outp[base + e] = static_cast<int32_t>(fget(cur, e).x);
                __syncthreads();
                break;
            }
            // Q_{j+1} = Q_j: keep the frontier in place and count digit j+1.
            for_each4(cur, n, [&](const uint2 (&it)[4], const bool (&v)[4]) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint64_t m = __ballot(v[u]);
                    if (m) hist_add(hn, digit(j + 1, it[u].y), v[u], m);
                }
            });
            __syncthreads();
            uint32_t* th = hc; hc = hn; hn = th;
            continue;
        }
        for_each4(cur, n, [&](const uint2 (&it)[4], const bool (&v)[4]) {
            bool take[4], keep[4];
            uint32_t idx[4], key[4], bin[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t d = digit(j, it[u].y);
                idx[u] = it[u].x;
                key[u] = it[u].y;
                take[u] = v[u] && (last && exact_fill ? d <= b : d < b);
                keep[u] = v[u] && d == b && !last;
                bin[u] = last ? 0u : digit(j + 1, it[u].y);
            }
            if (last && !exact_fill) {
                // Final digit: the boundary group holds equal keys; take the
                // first `need` of them in reservation order.
                bool tie[4];
                uint64_t m[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    tie[u] = v[u] && digit(j, it[u].y) == b;
                    m[u] = __ballot(tie[u]);
                }
                const uint64_t any = m[0] | m[1] | m[2] | m[3];
                if (any) {
                    uint32_t tot = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) tot += __builtin_popcountll(m[u]);
                    uint32_t base = wave_reserve(&sm.tie_cnt, any, tot);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (tie[u] && base + mbcnt(m[u]) < need) take[u] = true;
                        base += __builtin_popcountll(m[u]);
                    }
                }
            }
            commit4(take, idx, outp, k, sm);
            if (!last) append4(keep, idx, key, bin, nxt, hn);
        });
        __syncthreads();
        if (last) break;
        kq = need;
        const Frontier tf = cur; cur = nxt; nxt = tf;
        uint32_t* th = hc; hc = hn; hn = th;
    }
}

// Copies the wave frontiers (LDS share, then spill range) into one
// contiguous frontier dst, counts the leading digit of every key in h (any
// contents on entry) and returns whether all of its keys are equal
// (block-uniform; ends with a barrier).
__device__ __forceinline__ bool compact_waves(const uint2* spill_base, int64_t spill_len,
                                              uint2* dst, uint32_t* h, Shared& sm) {
    clear_hist(h);
    if (threadIdx.x == 0) {
        uint32_t o = 0;
        for (int w = 0; w < kWaves; ++w) { sm.offs[0][w] = o; o += sm.wcnt[w]; }
        sm.offs[0][kWaves] = o;
        sm.kext[0] = kNoElem;
        sm.kext[1] = 0;
    }
    __syncthreads();
    const uint32_t C = sm.offs[0][kWaves];
    uint32_t mn = kNoElem, mx = 0;
    for (uint32_t g = threadIdx.x; g < C; g += kBlock) {
        uint32_t w = 0;
        while (w + 1 < kWaves && sm.offs[0][w + 1] <= g) ++w;
        const uint32_t e = g - sm.offs[0][w];
        uint2 v;
        if (e < kWaveCap) {
            v = sm.front[w * kWaveCap + e];
        } else {
            const u32x2 t = nt_load2(spill_base + w * spill_len + (e - kWaveCap));
            v = make_uint2(t.x, t.y);
        }
        v.y = desc_key(v.y);
        nt_store2(dst + g, v.x, v.y);
        hist_add(h, v.y >> 21, true, __ballot(true));
        mn = v.y < mn ? v.y : mn;
        mx = v.y > mx ? v.y : mx;
    }
    lds_extremes(&sm.kext[0], mn, mx);
    __syncthreads();
    return sm.kext[0] == sm.kext[1];
}

// Phase 3 for a wave-private frontier of C entries (sizes in sm.wcnt, visible),
// quota kq, sm.out_cnt indices already committed; h1, h0: two 2048-bin LDS
// histograms (any contents).  When every wave's share fits on chip the
// frontier is refined from registers; otherwise it is gathered into `contig`
// (counting the leading digit) and refined through ping-pong buffers (LDS,
// then `spare`).  spill_base/spill_len locate the wave spills; `spare` may
// overlap them.
__device__ __forceinline__ void finish_waves(uint32_t C, const uint2* spill_base,
                                             int64_t spill_len, uint2* contig, uint2* spare,
                                             uint32_t* h1, uint32_t* h0, uint32_t kq,
                                             int32_t* outp, uint32_t k, Shared& sm) {
    const uint32_t out_base = sm.out_cnt;
    uint32_t wmax = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wmax = sm.wcnt[w] > wmax ? sm.wcnt[w] : wmax;
    if (wmax <= static_cast<uint32_t>(kWaveCap)) {
        const uint32_t mine = sm.wcnt[wave()];
        const uint2* reg = sm.front + wave() * kWaveCap;
        refine_regs<kWaveRegs>(
            [&](int u, uint32_t& i, uint32_t& key) {
                const uint32_t e = lane() + 64 * u;
                const bool on = e < mine;
                const uint2 v = reg[on ? e : 0u];
                i = v.x;
                key = desc_key(v.y);
                return on;
            },
            h1, h0, kq, out_base, outp, k, sm);
        return;
    }
    if (compact_waves(spill_base, spill_len, contig, h1, sm)) {
        // Every entry carries the same key (a constant row, say): no value
        // outside the frontier ranks above it, so its first kq entries are
        // the rest of the answer.
        for (uint32_t j = threadIdx.x; j < kq; j += kBlock) outp[out_base + j] = static_cast<int32_t>(contig[j].x);
        return;
    }
    if (threadIdx.x == 0) sm.cnt[0] = C;
    __syncthreads();
    const Frontier cur{sm.front, 0, contig, &sm.cnt[0]};
    const Frontier nxt{sm.front, kCapA, spare, &sm.cnt[1]};
    refine(cur, nxt, h1, h0, kq, outp, k, sm);
}

// Number of view samples and the view's phase for a row.
template <int S>
__device__ __forceinline__ uint32_t view_size(uint32_t row, uint32_t L, uint32_t* a) {
    *a = view_phase(row, S);
    return L > *a ? (L - *a + S - 1) / S : 0u;
}

__device__ __forceinline__ uint32_t clamp_len(int32_t v, int32_t n) {
    return static_cast<uint32_t>(v < 0 ? 0 : (v > n ? n : v));
}

// The row a persistent worker takes next, its valid length and, when its
// view is usable, the first batch of its view samples (loaded ahead).
struct NextRow {
    int row;
    uint32_t L;
    bool looked;
    uint32_t vb[kSampleVec];  // when looked: the row's first batch of view samples
};

// Ticket of the persistent queue (Sec. 5.5 "Persistent sampled").  A launch
// draws exactly M_live tickets, 0 .. M_live - 1, in the queue's modification
// order: every row taken draws one, and the one drawn for a workgroup's last
// row ends its loop.  The draw of ticket M_live - 1 is therefore the last
// access of the launch to the queue, and that workgroup returns it to zero; no
// other ordering is needed.  Thread 0 only.
//
// The queue serves rows [W, M_live) from the last one down (W = the pool
// size; the first wave takes rows 0 .. W - 1): in causal prefill a row's
// length grows with its index, so the longest rows go first and the rows
// still running when the queue is empty are the shortest.  Returns M_live for
// no row.
__device__ __forceinline__ int publish_ticket(const Params& p, uint32_t t, int m_live, Shared& sm) {
    if (t + 1 == static_cast<uint32_t>(m_live)) atomicExch(p.counters, 0u);
    const int left = m_live - static_cast<int>(gridDim.x);
    const int rn = static_cast<int>(t) < left ? m_live - 1 - static_cast<int>(t) : m_live;
    sm.next_row = rn;
    return rn;
}

// One row, whole-row ownership (persistent mapping).  L is the row's valid
// length; `looked`: vb holds the row's first batch of view samples, loaded
// when the previous row was done.  Thread 0 holds ticket t, drawn when the
// row started.  sliceA holds the wave spills, sliceB is the contiguous
// frontier of the general path.  On the sampled route the next row is
// published at the end of Phase 1, its length is read while this row
// streams, and its first batch of view samples is loaded when this row is
// done; nr.row < 0 means the next row is not known yet.
template <int S, bool DUAL, bool HINT>
__device__ __forceinline__ NextRow select_row(const Params& p, int row, uint32_t L, bool looked,
                                              const uint32_t (&vb)[kSampleVec], uint32_t t,
                                              int m_live, Shared& sm, uint2* sliceA,
                                              uint2* sliceB) {
    const uint32_t k = p.k;
    NextRow nr;
    nr.row = -1;
    nr.L = 0;
    nr.looked = false;
    int32_t* outp = p.out + static_cast<int64_t>(row) * k;
    if (L <= k) {
        sentinel_row(outp, L, k);
        count_route(p, TOPKF_ROUTE_SENTINEL);
        return nr;
    }
    const float* x = p.logits + static_cast<int64_t>(row) * p.stride;
    const int64_t wsl = wave_spill_len(p.n);
    uint32_t* h0 = sm.hist[0];
    uint32_t* h1 = sm.hist[1];
    WaveFrontier wf{sm.front + wave() * kWaveCap, sliceA + wave() * wsl, 0};
    int route = TOPKF_ROUTE_EXACT_DIRECT;
    bool certified = false;
    bool done = false;  // refined from the registers loaded at the publish
    uint32_t C = 0;
    uint32_t na = 0, nnv = 0;  // the next row's view
    const float* xn = nullptr;
    uint32_t vnext0 = kNoElem;  // its first sample per thread
    if constexpr (S > 0) {
        uint32_t a;
        const uint32_t nv = view_size<S>(row, L, &a);
        const uint32_t q = q_primary(k, S, p.prim_q), q1 = DUAL ? q_secondary(k, S, p.band_q) : q;
        uint32_t hkey = 0;
        bool hinted = false;
        if constexpr (HINT) hinted = row_hint(p, static_cast<uint32_t>(row), &hkey);
        if (hinted || nv >= q1) {
            uint32_t T0 = 0, T1 = 0;
            int32_t ke_next = 0;
            bool on = false;
            // h0 is clear (every row leaves it so).  Samples loaded ahead have
            // long arrived: they are counted before the row's first loads are
            // issued, so that counting them waits for nothing else.
            if (!hinted && looked) view_count(vb, h0);
            uint32_t vfirst[kSampleVec];
            const Span sp = make_span(x, 0, L);
            scan_span2<kScanVec>(
                sp,
                [&]() {
                    if (!hinted && !looked) view_batch(x, a, nv, S, 0u, vfirst);
                },
                [&]() {
                    if (threadIdx.x == 0) sm.out_cnt = 0;
                    if (hinted) {
                        T0 = hkey;  // the proposal replaces Phase 1; no band
                        T1 = hkey;
                        __syncthreads();
                    } else {
                        if (!looked) view_count(vfirst, h0);
                        const Cuts c = phase1(x, a, nv, S, q, q1, h0, sm, nullptr,
                                              static_cast<uint32_t>(kBlock * kSampleVec));
                        T0 = c.t0;
                        T1 = c.t1;
                    }
                    // The next row, drawn when this row started, is published
                    // now: the draw's latency hid behind Phase 1.
                    if (threadIdx.x == 0) publish_ticket(p, t, m_live, sm);
                    __syncthreads();
                    nr.row = sm.next_row;
                    if (nr.row < m_live) ke_next = p.ke[nr.row];
                },
                // a cutoff value >= +0 (T0 <= 0x7FFFFFFF) takes the raw compare
                [&]() { return T0 <= 0x7FFFFFFFu; },
                [&](u32x4 b, uint32_t i0) { admit4_raw(b, i0, T0 ^ 0x7FFFFFFFu, wf); },
                [&](u32x4 b, uint32_t i0) { admit4<false>(b, i0, 0u, T0, wf); },
                [&]() {
                    // The next row's geometry (its length has arrived by now).
                    nr.L = nr.row < m_live ? clamp_len(ke_next, p.n) : 0u;
                    if (nr.L > k) {
                        nnv = view_size<S>(static_cast<uint32_t>(nr.row), nr.L, &na);
                        on = !HINT && nnv >= q1;  // hinted launches load views inline
                        xn = p.logits + static_cast<int64_t>(nr.row) * p.stride;
                    }
                });
            nr.looked = on;
            // The next row's first view sample per thread goes out now, ahead
            // of this row's refinement, so that it has arrived when that row
            // starts counting its view (the rest of a longer view follows at
            // the end of this row).
            // Nothing this wave issued is still in flight here; the explicit
            // wait says so, and without it the compiler waits for this load
            // as soon as a register of the scan's ring is reused.
            __builtin_amdgcn_s_waitcnt(0);
            if (on) vnext0 = threadIdx.x < nnv ? __float_as_uint(xn[na + threadIdx.x * S]) : kNoElem;
            {
                // Each wave loads its own frontier share into registers as
                // soon as its scan is done (other waves may still be
                // scanning) and puts its keys' range next to its size: a
                // certified row on the primary route refines from these
                // registers in that range, with no load, reduction or barrier
                // of its own.
                uint32_t pidx[kWaveRegs], pkey[kWaveRegs];
                uint32_t pact = 0;
                const uint2* reg = sm.front + wave() * kWaveCap;
                const uint32_t mine = readfirst(wf.n);
                uint32_t mn = kNoElem, mx = 0;
#pragma unroll
                for (int u = 0; u < kWaveRegs; ++u) {
                    const uint32_t e = lane() + 64 * u;
                    const bool in = e < mine;
                    const uint2 v = reg[in ? e : 0u];
                    pidx[u] = v.x;
                    pkey[u] = desc_key(v.y);
                    pact |= in ? 1u << u : 0u;
                    mn = in && pkey[u] < mn ? pkey[u] : mn;
                    mx = in && pkey[u] > mx ? pkey[u] : mx;
                }
                mn = wave_min(mn);
                mx = wave_max(mx);
                if (lane() == 0) {
                    sm.wext[0][wave()] = mn;
                    sm.wext[1][wave()] = mx;
                }
                clear_hist(h1);
                C = publish_waves(wf, sm);
                uint32_t wmax = 0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) wmax = sm.wcnt[w] > wmax ? sm.wcnt[w] : wmax;
                if (C >= k && wmax <= static_cast<uint32_t>(kWaveCap)) {
                    if (hinted) count_route(p, TOPKF_ROUTE_HINTED);
                    count_route(p, TOPKF_ROUTE_PRIMARY);
                    const uint4* we = reinterpret_cast<const uint4*>(&sm.wext[0][0]);
                    const uint4 a = we[0], b = we[1], c = we[2], d = we[3];
                    const uint32_t lo = min(min(min(a.x, a.y), min(a.z, a.w)), min(min(b.x, b.y), min(b.z, b.w)));
                    const uint32_t hi = max(max(max(c.x, c.y), max(c.z, c.w)), max(max(d.x, d.y), max(d.z, d.w)));
                    refine_regs<kWaveRegs, true>(
                        [&](int u, uint32_t& i, uint32_t& key) {
                            i = pidx[u];
                            key = pkey[u];
                            return ((pact >> u) & 1u) != 0;
                        },
                        h1, h0, k, sm.out_cnt, outp, k, sm, lo, hi);
                    done = true;
                }
            }
            route = TOPKF_ROUTE_PRIMARY;
            if (!done && C < k) {
                route = TOPKF_ROUTE_EXACT_UNDERFILL;
                if (DUAL && T1 > T0) {
                    scan_span<kRowVec>(sp, NoPre{}, [&](u32x4 b, uint32_t i0) {
                        admit4<true>(b, i0, T0, T1, wf);
                    });
                    __syncthreads();
                    C = publish_waves(wf, sm);
                    if (C >= k) route = TOPKF_ROUTE_BAND;
                    // Drained here, so that no load of this pass is still
                    // counted where the code paths meet again: otherwise the
                    // compiler makes the primary route's refinement wait for
                    // the next row's view load (issued above) before it starts.
                    __builtin_amdgcn_s_waitcnt(0);
                }
            }
            certified = C >= k;
            if (hinted && !done) count_route(p, TOPKF_ROUTE_HINTED);
        }
    }
    if (!done) {
        uint32_t kq = k;
        if (!certified) {
            // The no-view plan serves short rows: keep them in registers.
            kq = exact_route<S == 0>(x, L, k, outp, wf, h0, sm);
            C = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) C += sm.wcnt[w];
        }
        count_route(p, route);
        bool spill = false;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) spill |= sm.wcnt[w] > static_cast<uint32_t>(kWaveCap);
        if (spill) count_route(p, TOPKF_ROUTE_SPILL);
        finish_waves(C, sliceA, wsl, sliceB, sliceA, h1, h0, kq, outp, k, sm);
    }
    clear_hist(h0);  // for the next row's view (made visible by the caller's barrier)
    // The next row's first batch of view samples goes out now, so that it has
    // arrived when that row starts, and the sampled lines are still cached
    // when its scan reads them.
    if constexpr (S > 0) {
        if (nr.looked) {
            nr.vb[0] = vnext0;
#pragma unroll
            for (int u = 1; u < kSampleVec; ++u) {
                const uint32_t j = u * kBlock + threadIdx.x;
                nr.vb[u] = j < nnv ? __float_as_uint(xn[na + j * S]) : kNoElem;
            }
        }
    }
    return nr;
}

template <int S, bool DUAL, bool HINT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void persistent_kernel(Params p) {
    __shared__ Shared sm;
    const int m_live = static_cast<int>(clamp_len(*p.num_valid_rows, p.m_cap));
    uint2* sliceA = p.ws + 2 * static_cast<int64_t>(blockIdx.x) * slice_len(p.n);
    uint2* sliceB = sliceA + slice_len(p.n);
    // First wave: workgroup w takes row w; afterwards rows come from the
    // queue.  The ticket of the next row is drawn when a row starts, so the
    // next row and its length are known during this row's Phase 1.
    int row = blockIdx.x;
    // The first row's length is loaded alongside the live-row count.
    const int32_t ke0 = row < p.m_cap ? p.ke[row] : 0;
    uint32_t L = row < m_live ? clamp_len(ke0, p.n) : 0u;
    bool looked = false;
    uint32_t vb[kSampleVec];
#pragma unroll
    for (int u = 0; u < kSampleVec; ++u) vb[u] = kNoElem;
    wave_priority(1);
    clear_hist(sm.hist[0]);  // the first row's view histogram
    __syncthreads();
    while (row < m_live) {
        uint32_t t = 0;
        if (threadIdx.x == 0) t = atomicAdd(p.counters, 1u);
        NextRow nr = select_row<S, DUAL, HINT>(p, row, L, looked, vb, t, m_live, sm, sliceA, sliceB);
        if (nr.row < 0) {  // routes without a view publish the ticket here
            if (threadIdx.x == 0) publish_ticket(p, t, m_live, sm);
            __syncthreads();
            nr.row = sm.next_row;
            nr.L = nr.row < m_live ? clamp_len(p.ke[nr.row], p.n) : 0u;
            nr.looked = false;
        }
        __syncthreads();
        row = nr.row;
        L = nr.L;
        looked = nr.looked;
#pragma unroll
        for (int u = 0; u < kSampleVec; ++u) vb[u] = nr.vb[u];
    }
}

// Bounds of part `part` of Pr near-equal contiguous segments of [0, L),
// aligned to 4 elements (Sec. 4.5: disjoint contiguous segments).
__device__ __forceinline__ uint32_t segment_chunk(uint32_t L, uint32_t Pr) {
    return ceil_div(ceil_div(L, Pr), 4) * 4;
}

// KV-split mapping (Sec. 4.5, Eqs. 26-27; Sec. 5.5 "Sampled KV-split"), as
// two kernels on the same stream.  kvsplit_scan_kernel: P workgroups per row
// each rebuild the row's view, derive the same tau0/tau1 and scan one
// contiguous segment, writing the admitted (index, key) pairs into the
// segment's own range of the row's region (primary candidates upward from
// the segment start, band candidates T0 < key <= T1 downward from its end)
// and their two counts, with the key range of its stored primary candidates.
// kvsplit_finish_kernel: one workgroup per row sums the counts (Eq. 27) and
// the key ranges, loads the candidates into registers and refines them in
// that range.  The kernel boundary makes every part's writes visible to the
// finisher on any XCD without per-workgroup cache write-back.
// Workgroups are numbered so that the parts of a row sit on one XCD (the
// dispatcher deals workgroup ids round-robin over the 8 XCDs), which keeps the
// replicated view reads in that XCD's L2.

struct RowGeom {
    uint32_t row, L, a, nv, q, q1, Pr, chunk;
    bool usable;
};

// Everything both KV-split kernels derive from (row, ke[row]) alone.
template <int S, bool DUAL>
__device__ __forceinline__ RowGeom kv_geom(const Params& p, uint32_t row, int32_t ke_row) {
    RowGeom g{};
    g.row = row;
    g.L = clamp_len(ke_row, p.n);
    g.usable = false;
    if constexpr (S > 0) {
        g.nv = view_size<S>(row, g.L, &g.a);
        g.q = q_primary(p.k, S, p.prim_q);
        g.q1 = DUAL ? q_secondary(p.k, S, p.band_q) : g.q;
        g.usable = g.nv >= g.q1;
    }
    uint32_t Pr = ceil_div(g.L > 0 ? g.L : 1u, static_cast<uint32_t>(p.min_seg));
    const uint32_t P = static_cast<uint32_t>(p.splits);
    g.Pr = Pr > P ? P : (Pr < 1 ? 1 : Pr);
    g.chunk = segment_chunk(g.L, g.Pr);
    return g;
}

__device__ __forceinline__ uint2* kv_region(const Params& p, uint32_t row) {
    return p.ws + 2 * static_cast<int64_t>(row) * slice_len(p.n);
}

// Per row, two words per part: its primary and band candidate counts.
__device__ __forceinline__ uint32_t* kv_counts(const Params& p, uint32_t row) {
    return reinterpret_cast<uint32_t*>(p.ws + 2 * static_cast<int64_t>(p.m_cap) * slice_len(p.n)) +
           2 * static_cast<int64_t>(row) * p.splits;
}

// After every row's counts, two words per part: the smallest and largest key
// among its stored primary candidates (kNoElem and 0 when it stored none).
__device__ __forceinline__ uint32_t* kv_ext(const Params& p, uint32_t row) {
    return kv_counts(p, 0) + 2 * static_cast<int64_t>(p.m_cap) * p.splits +
           2 * static_cast<int64_t>(row) * p.splits;
}

// Whole-row exact coarse route by one workgroup (rows without a usable view,
// and rows whose parts underfill even with the band).
__device__ __forceinline__ void kv_exact_row(const Params& p, const RowGeom& g, int route,
                                             Shared& sm) {
    const uint32_t k = p.k;
    int32_t* outp = p.out + static_cast<int64_t>(g.row) * k;
    const float* x = p.logits + static_cast<int64_t>(g.row) * p.stride;
    uint2* region = kv_region(p, g.row);
    uint2* region2 = region + slice_len(p.n);
    const int64_t wsl = wave_spill_len(p.n);
    WaveFrontier wf{sm.front + wave() * kWaveCap, region + wave() * wsl, 0};
    const uint32_t kq = exact_route<true>(x, g.L, k, outp, wf, sm.hist[0], sm);
    uint32_t C = 0;
    bool spill = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        C += sm.wcnt[w];
        spill |= sm.wcnt[w] > static_cast<uint32_t>(kWaveCap);
    }
    count_route(p, route);
    if (spill) count_route(p, TOPKF_ROUTE_SPILL);
    finish_waves(C, region, wsl, region2, region, sm.hist[1], sm.hist[0], kq, outp, k, sm);
}

template <int S, bool DUAL, bool HINT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void kvsplit_scan_kernel(Params p) {
    __shared__ Shared sm;
    const uint32_t P = static_cast<uint32_t>(p.splits);
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t li = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const uint32_t row = li / P, part = li % P;
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    // Both loads in flight at once (ke has M_cap entries).
    const int32_t nvr = *p.num_valid_rows;
    const int32_t ke_row = p.ke[row];
    uint32_t hkey = 0;
    bool hinted = false;
    if constexpr (HINT) hinted = row_hint(p, row, &hkey);
    const uint32_t m_live = clamp_len(nvr, p.m_cap);
    if (row >= m_live) return;
    const uint32_t k = p.k;
    const RowGeom g = kv_geom<S, DUAL>(p, row, ke_row);
    if (g.L <= k) {
        if (part == 0) {
            sentinel_row(p.out + static_cast<int64_t>(row) * k, g.L, k);
            count_route(p, TOPKF_ROUTE_SENTINEL);
        }
        return;
    }
    if (!g.usable && !hinted) {
        // No usable view: part 0 runs the exact coarse route over the whole row.
        if (part == 0) kv_exact_row(p, g, TOPKF_ROUTE_EXACT_DIRECT, sm);
        return;
    }
    if (part >= g.Pr) return;
    const uint32_t L = g.L;
    const uint32_t lo = part * g.chunk < L ? part * g.chunk : L;
    const uint32_t hi = lo + g.chunk < L ? lo + g.chunk : L;
    const float* x = p.logits + static_cast<int64_t>(row) * p.stride;
    uint2* region = kv_region(p, row);
    uint32_t* h0 = sm.hist[0];

    // Phases 1 and 2 for this part.  The view samples are loaded first and
    // awaited before the segment's loads go out: issued together, the
    // samples queue behind every part's segment loads in the memory system
    // and Phase 1 waits for the whole flood (measured on decode: samples
    // complete 6 us after launch).  The segment's first chunk is then in
    // flight while the (replicated) view is histogrammed.
    uint32_t T0 = 0, T1 = 0;
    // Candidates are staged in the wave's share of the LDS frontier with
    // wave-uniform counts (primary from the bottom, band from the top) and
    // written out once per wave after the scan; a wave whose share fills up
    // writes the rest straight to its reserved slots.
    uint2* stg = sm.front + wave() * kWaveCap;
    uint32_t sp_n = 0, sb_n = 0;
    uint32_t pmin = kNoElem, pmax = 0;  // keys of primary candidates written directly
    uint32_t vb[kSampleVec];
    const Span sp = make_span(x, lo, hi);
    uint32_t vt0 = 0;         // raw admission: signed-int form of the cutoff
    int mode = 0;             // 0: raw compare, 1: key compare, 2: key compare with flood control
    uint32_t full[2] = {kNoElem, kNoElem};
    // The element step, in three compiled forms so that each part runs a
    // straight-line scan with only the code its mode needs.  RAW: the cutoff
    // value is >= +0 and admission is the signed compare of admit4_raw.
    // FLOOD: the view put many times the target sample count at or above the
    // cutoff (a constant or heavily tied row); a wave whose stage is full then
    // also tracks a flood key per part and kind (below).
    auto step = [&](auto raw_c, auto flood_c) {
        constexpr bool RAW = decltype(raw_c)::value;
        constexpr bool FLOOD = decltype(flood_c)::value;
        return [&](u32x4 b, uint32_t i0) {
            if constexpr (FLOOD) {
                // Once this part holds K stored copies of its primary flood
                // value, a step whose every element carries that bit pattern
                // would only be left out below: skip it outright.
                if (full[0] != kNoElem) {
                    const uint32_t fb = bits_of_key(full[0]);
                    const bool same = b[0] == fb && b[1] == fb && b[2] == fb && b[3] == fb;
                    if (__builtin_amdgcn_ballot_w64(!same) == 0) return;
                }
            }
            uint32_t key[4];
            bool pp[4], pb[4];
            uint64_t mp[4], mb[4];
            uint32_t tp = 0, tb = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if constexpr (RAW) {
                    pp[u] = static_cast<int32_t>(b[u]) >= static_cast<int32_t>(vt0);
                    key[u] = b[u] ^ 0x7FFFFFFFu;  // desc_key of a value >= +0
                    pb[u] = false;
                } else {
                    key[u] = desc_key(b[u]);
                    pp[u] = key[u] <= T0;
                    pb[u] = DUAL && key[u] > T0 && key[u] <= T1;
                }
                mp[u] = __builtin_amdgcn_ballot_w64(pp[u]);
                mb[u] = (DUAL && !RAW) ? __builtin_amdgcn_ballot_w64(pb[u]) : 0ull;
                tp += __builtin_popcountll(mp[u]);
                tb += __builtin_popcountll(mb[u]);
            }
            if (sp_n + sb_n + tp + tb <= static_cast<uint32_t>(kWaveCap)) {
                // Staged in the wave's LDS share: primary upward, band downward.
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (pp[u]) stg[mbcnt_from(mp[u], sp_n)] = make_uint2(i0 + u, key[u]);
                    sp_n += __builtin_popcountll(mp[u]);
                    if (DUAL && !RAW) {
                        if (pb[u]) stg[kWaveCap - 1 - mbcnt_from(mb[u], sb_n)] = make_uint2(i0 + u, key[u]);
                        sb_n += __builtin_popcountll(mb[u]);
                    }
                }
                return;
            }
            if constexpr (FLOOD) {
                if (tp + tb >= 128u) {
                    // Admission in bulk.  The key of the batch's first
                    // candidate is tracked per part and kind; once the part
                    // holds K stored copies of it, further copies are counted
                    // out rather than stored.  Exact: any K equal keys are an
                    // answer at a boundary (Sec. 4.4), and a copy left out has
                    // K stored copies of its value, so the K-th largest of the
                    // stored candidates and every candidate above it are those
                    // of all the candidates; a part that leaves one out holds
                    // >= K, so certification decides as before.
                    uint64_t mm[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) mm[u] = mp[u] | mb[u];
                    const int uf = mm[0] ? 0 : mm[1] ? 1 : mm[2] ? 2 : 3;
                    const uint32_t lf = static_cast<uint32_t>(__builtin_ctzll(mm[uf]));
                    const uint32_t kv = uf == 0 ? key[0] : uf == 1 ? key[1] : uf == 2 ? key[2] : key[3];
                    const uint32_t kf = static_cast<uint32_t>(
                        __builtin_amdgcn_readlane(static_cast<int>(kv), static_cast<int>(lf)));
                    const int kind = (mp[uf] >> lf) & 1ull ? 0 : 1;
                    bool eq[4];
                    uint64_t me[4];
                    uint32_t ne = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        eq[u] = (kind ? pb[u] : pp[u]) && key[u] == kf;
                        me[u] = __builtin_amdgcn_ballot_w64(eq[u]);
                        ne += __builtin_popcountll(me[u]);
                    }
                    if (ne >= 64u && kf != kNoElem) {
                        // full[kind]: a key this wave already saw reach K
                        // stored copies in the part (the count only grows)
                        uint32_t drop = kf == full[kind] ? 1u : 0u;
                        if (!drop) {
                            if (lane() == 0) {
                                const uint32_t cur = atomicCAS(&sm.fkey[kind], kNoElem, kf);
                                if (cur == kNoElem || cur == kf) drop = atomicAdd(&sm.fcnt[kind], ne) >= k;
                            }
                            drop = readlane(drop, 0);
                            if (drop) full[kind] = kf;
                        }
                        if (drop) {
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                if (kind) { pb[u] = pb[u] && !eq[u]; mb[u] &= ~me[u]; }
                                else { pp[u] = pp[u] && !eq[u]; mp[u] &= ~me[u]; }
                            }
                            if (kind) tb -= ne; else tp -= ne;
                            if (tp + tb == 0) return;
                        }
                    }
                }
            }
            // kind 0: primary, upward from lo; kind 1: band, downward from hi - 1
            auto emit = [&](const bool (&pr)[4], int kind) {
                uint64_t m[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) m[u] = __ballot(pr[u]);
                const uint64_t any = m[0] | m[1] | m[2] | m[3];
                if (any == 0) return;
                uint32_t tot = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) tot += __builtin_popcountll(m[u]);
                uint32_t base = wave_reserve(&sm.cnt[kind], any, tot);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (pr[u]) {
                        const uint32_t slot = base + mbcnt(m[u]);
                        region[kind ? hi - 1 - slot : lo + slot] = make_uint2(i0 + u, key[u]);
                        if (kind == 0) {
                            pmin = key[u] < pmin ? key[u] : pmin;
                            pmax = key[u] > pmax ? key[u] : pmax;
                        }
                    }
                    base += __builtin_popcountll(m[u]);
                }
            };
            emit(pp, 0);
            if (DUAL && !RAW) emit(pb, 1);
        };
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // Dual-boundary plans have no raw form and no flood form: their band
    // makes a second classification per score, and three chunk loops in one
    // kernel spill registers.
    scan_span_sel<kSegVec, DUAL ? 1 : 3>(
        sp,
        [&]() {
            if (!hinted) {
                view_batch(x, g.a, g.nv, S, 0u, vb);
                __builtin_amdgcn_s_waitcnt(0);
            }
        },
        [&]() {
            clear_hist(h0);
            if (threadIdx.x == 0) {
                sm.cnt[0] = 0;
                sm.cnt[1] = 0;
                sm.kext[0] = kNoElem;
                sm.kext[1] = 0;
                sm.fkey[0] = kNoElem;
                sm.fkey[1] = kNoElem;
                sm.fcnt[0] = 0;
                sm.fcnt[1] = 0;
            }
            __syncthreads();
            bool flood = false;
            if (hinted) {
                T0 = hkey;  // the proposal replaces Phase 1; no band
                T1 = hkey;
            } else {
                const Cuts c = phase1(x, g.a, g.nv, S, g.q, g.q1, h0, sm, vb);
                T0 = c.t0;
                T1 = c.t1;
                // samples at or above the primary boundary's coarse bin
                const uint32_t b0 = readfirst(sm.res[0]);
                flood = readfirst(sm.res[1]) + readfirst(h0[b0]) > 8u * g.q;
            }
            vt0 = T0 ^ 0x7FFFFFFFu;
            mode = DUAL ? 1 : flood ? 2 : T0 <= 0x7FFFFFFFu ? 0 : 1;
        },
        [&]() { return mode; },
        step(std::integral_constant<bool, !DUAL>{}, F_{}), step(F_{}, F_{}),
        step(F_{}, std::integral_constant<bool, !DUAL>{}),
        NoPre{});
    // Flush the staged entries: one reservation per wave and kind, then
    // coalesced stores.  Each wave reads back only its own share.  Plain
    // (cached) stores: the row's finisher runs on the same XCD and reads
    // them back from its L2 (nontemporal stores cost it 0.5 us on decode).
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (mode != 2) {
        uint32_t pbase = 0, bbase = 0;
        if (lane() == 0) {
            if (sp_n) pbase = atomicAdd(&sm.cnt[0], sp_n);
            if (DUAL && sb_n) bbase = atomicAdd(&sm.cnt[1], sb_n);
        }
        pbase = readlane(pbase, 0);
        bbase = readlane(bbase, 0);
        for (uint32_t e = lane(); e < sp_n; e += 64) {
            const uint2 v = stg[e];
            region[lo + pbase + e] = v;
        }
        if (DUAL) {
            for (uint32_t e = lane(); e < sb_n; e += 64) {
                const uint2 v = stg[kWaveCap - 1 - e];
                region[hi - 1 - (bbase + e)] = v;
            }
        }
    } else {
        // Staged copies of a flood key that already has K stored copies in
        // the part are left out as in the scan (the count only grows, so a
        // value read while other waves still scan is a valid lower bound).
        auto flush = [&](int kind, uint32_t n) {
            if (n == 0) return;
            const uint32_t dk = readfirst(sm.fcnt[kind]) >= k ? readfirst(sm.fkey[kind]) : kNoElem;
            auto at = [&](uint32_t e) { return stg[kind ? kWaveCap - 1 - e : e]; };
            uint32_t keep = n;
            if (dk != kNoElem) {
                keep = 0;
                for (uint32_t e0 = 0; e0 < n; e0 += 64) {
                    const uint32_t e = e0 + lane();
                    keep += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < n && at(e).y != dk));
                }
            }
            uint32_t base = 0;
            if (lane() == 0 && keep) base = atomicAdd(&sm.cnt[kind], keep);
            base = readlane(base, 0);
            for (uint32_t e0 = 0; e0 < n; e0 += 64) {
                const uint32_t e = e0 + lane();
                uint2 v = make_uint2(0u, dk);
                if (e < n) v = at(e);
                const bool kp = e < n && v.y != dk;
                const uint64_t m = __builtin_amdgcn_ballot_w64(kp);
                const uint32_t slot = base + mbcnt(m);
                if (kp) region[kind ? hi - 1 - slot : lo + slot] = v;
                base += __builtin_popcountll(m);
            }
        };
        flush(0, sp_n);
        if (DUAL) flush(1, sb_n);
    }
    // The part also publishes the key range of its stored primary candidates
    // ([kNoElem, 0] when it has none): the finisher's first digit window, and
    // a tail of equal keys recognised without reading it.  Staged copies of a
    // flood key left out above carry a key that is also stored, so they do
    // not change the range.
    for (uint32_t e = lane(); e < sp_n; e += 64) {
        const uint32_t key = stg[e].y;
        pmin = key < pmin ? key : pmin;
        pmax = key > pmax ? key : pmax;
    }
    lds_extremes(&sm.kext[0], pmin, pmax);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t* counts = kv_counts(p, row);
        counts[2 * part] = sm.cnt[0];
        counts[2 * part + 1] = sm.cnt[1];
        uint32_t* ext = kv_ext(p, row);
        ext[2 * part] = sm.kext[0];
        ext[2 * part + 1] = sm.kext[1];
    }
}

template <int S, bool DUAL, bool HINT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void kvsplit_finish_kernel(Params p) {
    __shared__ Shared sm;
    // same XCD as the row's parts in kvsplit_scan_kernel
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t row = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    // The live-row count, the row's length and the parts' counts and key
    // ranges (wave 0, four parts per lane) are loaded together; entries of
    // parts the row did not use this call are stale and are dropped below.
    const int32_t nvr = *p.num_valid_rows;
    const int32_t ke_row = p.ke[row];
    uint32_t hkey = 0;
    bool hinted = false;
    if constexpr (HINT) hinted = row_hint(p, row, &hkey);
    const uint32_t* counts = kv_counts(p, row);
    const uint32_t* exts = kv_ext(p, row);
    uint32_t c4[2][4], e4[2][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint32_t pp = 4 * lane() + v;
        c4[0][v] = 0;
        c4[1][v] = 0;
        e4[0][v] = kNoElem;
        e4[1][v] = 0;
        if (wave() == 0 && pp < static_cast<uint32_t>(p.splits)) {
            c4[0][v] = counts[2 * pp];
            c4[1][v] = counts[2 * pp + 1];
            e4[0][v] = exts[2 * pp];
            e4[1][v] = exts[2 * pp + 1];
        }
    }
    const uint32_t m_live = clamp_len(nvr, p.m_cap);
    if (row >= m_live) return;
    const uint32_t k = p.k;
    const RowGeom g = kv_geom<S, DUAL>(p, row, ke_row);
    if (g.L <= k || (!g.usable && !hinted)) return;  // finished by the scan kernel
    if (hinted) count_route(p, TOPKF_ROUTE_HINTED);
    const uint32_t L = g.L, Pr = g.Pr, chunk = g.chunk;
    int32_t* outp = p.out + static_cast<int64_t>(row) * k;
    uint2* region = kv_region(p, row);
    uint2* region2 = region + slice_len(p.n);
    uint32_t* h0 = sm.hist[0];
    uint32_t* h1 = sm.hist[1];

    // Merge the parts (Eq. 27): wave 0 forms the prefix offsets of the
    // primary and band counts, the largest count of one part and the key
    // range of the primary candidates; one barrier publishes them.
    if (wave() == 0) {
        uint32_t mxp = 0, kmn = kNoElem, kmx = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (4 * lane() + v < Pr) {
                kmn = e4[0][v] < kmn ? e4[0][v] : kmn;
                kmx = e4[1][v] > kmx ? e4[1][v] : kmx;
            }
        }
        kmn = wave_min(kmn);
        kmx = wave_max(kmx);
#pragma unroll
        for (int kind = 0; kind < 2; ++kind) {
            uint32_t s4 = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if (4 * lane() + v >= Pr) c4[kind][v] = 0;
                s4 += c4[kind][v];
                mxp = c4[kind][v] > mxp ? c4[kind][v] : mxp;
            }
            const uint32_t incl = wave_incl_scan(s4);
            uint32_t o = incl - s4;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t pp = 4 * lane() + v;
                if (pp < Pr) sm.offs[kind][pp] = o;
                o += c4[kind][v];
            }
            if (lane() == 63) sm.offs[kind][Pr] = incl;
        }
        mxp = wave_max(mxp);
        if (lane() == 0) {
            sm.part_max = mxp;
            sm.kext[0] = kmn;
            sm.kext[1] = kmx;
            sm.out_cnt = 0;
        }
    }
    clear_hist(h1);
    __syncthreads();  // offsets visible
    const uint32_t C0 = sm.offs[0][Pr], CB = sm.offs[1][Pr];
    int route = TOPKF_ROUTE_PRIMARY;
    uint32_t ctot = C0;
    if (C0 < k) {
        route = TOPKF_ROUTE_EXACT_UNDERFILL;
        if (DUAL && C0 + CB >= k) { route = TOPKF_ROUTE_BAND; ctot = C0 + CB; }
    }
    if (route == TOPKF_ROUTE_EXACT_UNDERFILL) {
        kv_exact_row(p, g, route, sm);
        return;
    }
    count_route(p, route);
    if (ctot <= static_cast<uint32_t>(kBlock * kRegs)) {
        const uint32_t klo = sm.kext[0], khi = sm.kext[1];
        // Register slots: when no part holds more than cap = 2^lc candidates
        // of a kind, with nr * cap <= kBlock * kRegs for the nr part ranges in
        // use, range q takes slots [q cap, (q + 1) cap) and a slot finds its
        // candidate by a shift and a mask.  Otherwise each slot locates its
        // candidate (the part p with off[p] <= r < off[p + 1]) with a
        // branch-free binary search over the LDS offsets.
        const uint32_t nr = route == TOPKF_ROUTE_BAND ? 2 * Pr : Pr;
        uint32_t lc = 13;
        while (lc > 0 && (nr << lc) > static_cast<uint32_t>(kBlock * kRegs)) --lc;
        uint32_t src[kRegs];
        bool live[kRegs];
        if (sm.part_max <= (1u << lc) && route == TOPKF_ROUTE_PRIMARY) {
            // Slot gq = tid + kBlock u: with kBlock = 2^9, its range is
            // (kBlock u) >> lc when lc >= 9 (the same for the whole block)
            // and (u << (9 - lc)) + (tid >> lc) otherwise, its position in
            // the range (kBlock u) & (cap - 1) + tid or tid & (cap - 1):
            // a per-thread part set once and a uniform part per slot.
            static_assert(kBlock == 512, "the slot split below assumes kBlock = 2^9");
            const uint32_t cap = 1u << lc;
            const bool wide = lc >= 9;
            const uint32_t tq = wide ? 0u : threadIdx.x >> lc;
            const uint32_t jt = wide ? threadIdx.x : threadIdx.x & (cap - 1u);
            const uint32_t tbase = tq * chunk + jt;
#pragma unroll
            for (int u = 0; u < kRegs; ++u) {
                const uint32_t qs = wide ? (static_cast<uint32_t>(kBlock) * u) >> lc
                                         : static_cast<uint32_t>(u) << (9 - lc);
                const uint32_t js = wide ? (static_cast<uint32_t>(kBlock) * u) & (cap - 1u) : 0u;
                const uint32_t q = qs + tq;
                const uint32_t* o = sm.offs[0] + (q < Pr ? q : 0u);
                const uint32_t n = o[1] - o[0];
                live[u] = (q < Pr) & (js + jt < n);
                src[u] = live[u] ? qs * chunk + js + tbase : 0u;
            }
        } else if (sm.part_max <= (1u << lc)) {
            // every LDS read unconditional, so that they issue together
#pragma unroll
            for (int u = 0; u < kRegs; ++u) {
                const uint32_t gq = threadIdx.x + kBlock * u;
                const uint32_t q = gq >> lc, j = gq & ((1u << lc) - 1u);
                const uint32_t kind = q >= Pr ? 1u : 0u;
                const uint32_t pp = q < nr ? q - kind * Pr : 0u;
                const uint32_t* o = sm.offs[kind] + pp;
                const uint32_t n = o[1] - o[0];
                live[u] = (q < nr) & (j < n);
                const uint32_t s0 = pp * chunk;
                const uint32_t s1 = s0 + chunk < L ? s0 + chunk : L;
                const uint32_t sv = kind ? s1 - 1 - j : s0 + j;
                src[u] = live[u] ? sv : 0u;
            }
        } else {
            uint32_t pstep = 1;
            while (pstep * 2 <= Pr) pstep *= 2;
#pragma unroll
            for (int u = 0; u < kRegs; ++u) src[u] = 0;
            for (uint32_t step = pstep; step > 0; step >>= 1) {
#pragma unroll
                for (int u = 0; u < kRegs; ++u) {
                    const uint32_t gi = threadIdx.x + kBlock * u;
                    const int kind = gi < C0 ? 0 : 1;
                    const uint32_t r = kind ? gi - C0 : gi;
                    const uint32_t cand = src[u] + step;
                    const uint32_t ov = sm.offs[kind][cand < Pr ? cand : 0u];
                    if (gi < ctot && cand < Pr && ov <= r) src[u] = cand;
                }
            }
#pragma unroll
            for (int u = 0; u < kRegs; ++u) {
                const uint32_t gi = threadIdx.x + kBlock * u;
                const int kind = gi < C0 ? 0 : 1;
                const uint32_t r = kind ? gi - C0 : gi;
                const uint32_t pp = src[u];
                const uint32_t ov = sm.offs[kind][pp];
                live[u] = gi < ctot;
                const uint32_t j = live[u] ? r - ov : 0u;
                const uint32_t s0 = pp * chunk;
                const uint32_t s1 = s0 + chunk < L ? s0 + chunk : L;
                const uint32_t sv = kind ? s1 - 1 - j : s0 + j;
                src[u] = live[u] ? sv : 0u;
            }
        }
        auto ld = [&](int u, uint32_t& i, uint32_t& key) {
            const uint2 t2 = region[src[u]];
            i = t2.x;
            key = t2.y;
            return live[u];
        };
        // the primary candidates' key range is the parts' published one
        if (route == TOPKF_ROUTE_PRIMARY) refine_regs<kRegs, true>(ld, h1, h0, k, 0u, outp, k, sm, klo, khi);
        else refine_regs<kRegs>(ld, h1, h0, k, 0u, outp, k, sm);
        return;
    }
    // Large frontier.  When every candidate carries the same key (a constant
    // row, say), no value outside them ranks above it, so any K of them are
    // the answer and refinement has nothing to separate; the first K in
    // offset order are taken.  On the primary route the parts' published key
    // extremes decide this; with the band, the extremes are read from the
    // candidates, range by range with several loads in flight.
    {
        uint32_t kmn = kNoElem, kmx = 0;
        if (threadIdx.x < Pr) {
            const uint32_t* ext = kv_ext(p, row);
            kmn = ext[2 * threadIdx.x];
            kmx = ext[2 * threadIdx.x + 1];
        }
        if (threadIdx.x == 0) { sm.kext[0] = kNoElem; sm.kext[1] = 0; }
        __syncthreads();
        lds_extremes(&sm.kext[0], kmn, kmx);  // the parts' published key ranges
        __syncthreads();
        bool tied = route == TOPKF_ROUTE_PRIMARY && sm.kext[0] == sm.kext[1];
        if (!tied) {
            __syncthreads();  // every thread has read the published extremes
            if (threadIdx.x == 0) { sm.kext[0] = kNoElem; sm.kext[1] = 0; }
            __syncthreads();
            uint32_t mn = kNoElem, mx = 0;
            const int kinds = route == TOPKF_ROUTE_BAND ? 2 : 1;
            for (int kind = 0; kind < kinds; ++kind) {
                for (uint32_t pp = 0; pp < Pr; ++pp) {
                    const uint32_t c = sm.offs[kind][pp + 1] - sm.offs[kind][pp];
                    const uint32_t s0 = pp * chunk;
                    const uint32_t s1 = s0 + chunk < L ? s0 + chunk : L;
                    for (uint32_t j0 = 0; j0 < c; j0 += 8 * kBlock) {
                        uint32_t kk[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const uint32_t j = j0 + u * kBlock + threadIdx.x;
                            kk[u] = kNoElem;
                            if (j < c) kk[u] = nt_load2(region + (kind ? s1 - 1 - j : s0 + j)).y;
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const uint32_t j = j0 + u * kBlock + threadIdx.x;
                            if (j < c) {
                                mn = kk[u] < mn ? kk[u] : mn;
                                mx = kk[u] > mx ? kk[u] : mx;
                            }
                        }
                    }
                }
            }
            lds_extremes(&sm.kext[0], mn, mx);
            __syncthreads();
            tied = sm.kext[0] == sm.kext[1];
        }
        if (tied) {
            for (uint32_t gi = threadIdx.x; gi < k; gi += kBlock) {
                const int kind = gi < C0 ? 0 : 1;
                const uint32_t r = kind ? gi - C0 : gi;
                const uint32_t* off = sm.offs[kind];
                uint32_t lo_p = 0, hi_p = Pr;  // the part with off[lo_p] <= r < off[lo_p + 1]
                while (hi_p - lo_p > 1) {
                    const uint32_t mid = (lo_p + hi_p) >> 1;
                    if (off[mid] <= r) lo_p = mid; else hi_p = mid;
                }
                const uint32_t j = r - off[lo_p];
                const uint32_t s0 = lo_p * chunk;
                const uint32_t s1 = s0 + chunk < L ? s0 + chunk : L;
                outp[gi] = static_cast<int32_t>(nt_load2(region + (kind ? s1 - 1 - j : s0 + j)).x);
            }
            return;
        }
    }
    // Otherwise gather the part ranges into one contiguous frontier (LDS,
    // then region2), count the leading digit, refine through ping-pong
    // buffers.
    const Frontier G{sm.front, kFront, region2, &sm.cnt[0]};
    for (uint32_t g0 = 0; g0 < ctot; g0 += 4 * kBlock) {
        uint2 it[4];
        bool v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t gi = g0 + u * kBlock + threadIdx.x;
            v[u] = gi < ctot;
            it[u] = make_uint2(0u, kNoElem);
            if (v[u]) {
                const int kind = gi < C0 ? 0 : 1;
                const uint32_t r = kind ? gi - C0 : gi;
                const uint32_t* off = sm.offs[kind];
                uint32_t lo_p = 0, hi_p = Pr;  // the part with off[pp] <= r < off[pp + 1]
                while (hi_p - lo_p > 1) {
                    const uint32_t mid = (lo_p + hi_p) >> 1;
                    if (off[mid] <= r) lo_p = mid; else hi_p = mid;
                }
                const uint32_t j = r - off[lo_p];
                const uint32_t s0 = lo_p * chunk;
                const uint32_t s1 = s0 + chunk < L ? s0 + chunk : L;
                const u32x2 t2 = nt_load2(region + (kind ? s1 - 1 - j : s0 + j));
                it[u] = make_uint2(t2.x, t2.y);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t gi = g0 + u * kBlock + threadIdx.x;
            if (v[u]) {
                fput(G, gi, it[u].x, it[u].y);
                lds_inc(h1, it[u].y >> 21);
            }
        }
    }
    if (threadIdx.x == 0) sm.cnt[0] = ctot;
    __syncthreads();
    count_route(p, TOPKF_ROUTE_SPILL);
    // General path: Q1 goes to global memory (the part ranges are consumed).
    const Frontier nxt{sm.front, 0, region, &sm.cnt[1]};
    refine(G, nxt, h1, h0, k, outp, k, sm);
}

// Cooperative exact coarse route (Sec. 5.5 "Eight-CTA exact cluster": with
// only a few long rows and no view, the row's segments go to several
// workgroups; without distributed shared memory their histograms merge in
// global memory).  Four kernels on the stream, the kernel boundaries making
// each step's global writes visible to the next:
//   kvx_hist_kernel      each part counts the coarse keys c(x) of its segment
//                        and adds its histogram into the row's histogram in
//                        the counter buffer;
//   kvx_cut_kernel       one workgroup per row reads (and clears) that
//                        histogram and finds tau* = min{b : C(b) >= K} and
//                        |E0| = C(tau* - 1) (Eq. 20);
//   kvx_classify_kernel  each part rescans its segment, committing c < tau*
//                        straight to the output and appending c == tau* to
//                        the row's frontier, through the row's two slot
//                        counters (staged per wave in LDS, one reservation per
//                        flush);
//   kvx_finish_kernel    one workgroup per row refines the frontier for the
//                        remaining K - |E0| slots and zeroes the row's counters.
// The commit predicate is the same device c(x) in both passes, so exactly
// |E0| indices are committed.

__device__ __forceinline__ uint32_t* kvx_hist(const Params& p, uint32_t row) {
    return p.counters + kCounterHead + 2 * static_cast<int64_t>(p.m_cap) +
           static_cast<int64_t>(row) * kBins;
}

__device__ __forceinline__ uint32_t* kvx_ctr(const Params& p, uint32_t row) {
    return p.counters + kCounterHead + 2 * static_cast<int64_t>(row);
}

// The (row, part) of a part workgroup (same numbering as the KV-split scan,
// the parts of a row on one XCD) and of a per-row workgroup.
__device__ __forceinline__ void kvx_part(const Params& p, uint32_t* row, uint32_t* part) {
    const uint32_t P = static_cast<uint32_t>(p.splits);
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t li = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    *row = li / P;
    *part = li % P;
}

__device__ __forceinline__ uint32_t kvx_row(void) {
    const uint32_t per_xcd = gridDim.x / 8;
    return (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void kvx_hist_kernel(Params p) {
    __shared__ Shared sm;
    uint32_t row, part;
    kvx_part(p, &row, &part);
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    const int32_t nvr = *p.num_valid_rows;
    const int32_t ke_row = p.ke[row];
    if (row >= clamp_len(nvr, p.m_cap)) return;
    const uint32_t k = p.k;
    const RowGeom g = kv_geom<0, false>(p, row, ke_row);
    if (g.L <= k) {
        if (part == 0) {
            sentinel_row(p.out + static_cast<int64_t>(row) * k, g.L, k);
            count_route(p, TOPKF_ROUTE_SENTINEL);
        }
        return;
    }
    if (part >= g.Pr) return;
    const uint32_t lo = part * g.chunk < g.L ? part * g.chunk : g.L;
    const uint32_t hi = lo + g.chunk < g.L ? lo + g.chunk : g.L;
    uint32_t* h = sm.hist[0];
    clear_hist(h);
    __syncthreads();
    const Span sp = make_span(p.logits + static_cast<int64_t>(row) * p.stride, lo, hi);
    scan_span<kSegVec>(sp, NoPre{}, [&](u32x4 b, uint32_t) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool v = b[u] != kNoElem;
            const uint64_t m = __ballot(v);
            if (m) hist_add(h, v ? coarse_of_bits(b[u]) : 0u, v, m);
        }
    });
    __syncthreads();
    uint32_t* gh = kvx_hist(p, row);
    const uint4 c = reinterpret_cast<const uint4*>(h)[threadIdx.x];
    const uint32_t b0 = 4 * threadIdx.x;
    if (c.x) atomicAdd(gh + b0, c.x);
    if (c.y) atomicAdd(gh + b0 + 1, c.y);
    if (c.z) atomicAdd(gh + b0 + 2, c.z);
    if (c.w) atomicAdd(gh + b0 + 3, c.w);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void kvx_cut_kernel(Params p) {
    __shared__ Shared sm;
    const uint32_t row = kvx_row();
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    const int32_t nvr = *p.num_valid_rows;
    const int32_t ke_row = p.ke[row];
    if (row >= clamp_len(nvr, p.m_cap)) return;
    if (clamp_len(ke_row, p.n) <= static_cast<uint32_t>(p.k)) return;
    // Read the merged histogram and return it to zero (this is its only reader).
    uint32_t* gh = kvx_hist(p, row);
    uint32_t* h = sm.hist[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = 4 * threadIdx.x + i;
        h[b] = gh[b];
        gh[b] = 0;
    }
    __syncthreads();
    const uint32_t t[1] = {static_cast<uint32_t>(p.k)};
    block_find<1>(h, t, sm);
    if (threadIdx.x == 0) {
        uint32_t* rec = kv_counts(p, row);
        rec[0] = sm.res[0];  // tau*
        rec[1] = sm.res[1];  // |E0| = C(tau* - 1)
    }
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void kvx_classify_kernel(Params p) {
    __shared__ Shared sm;
    uint32_t row, part;
    kvx_part(p, &row, &part);
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    const int32_t nvr = *p.num_valid_rows;
    const int32_t ke_row = p.ke[row];
    if (row >= clamp_len(nvr, p.m_cap)) return;
    const uint32_t k = p.k;
    const RowGeom g = kv_geom<0, false>(p, row, ke_row);
    if (g.L <= k || part >= g.Pr) return;
    const uint32_t tau = kv_counts(p, row)[0];
    const uint32_t lo = part * g.chunk < g.L ? part * g.chunk : g.L;
    const uint32_t hi = lo + g.chunk < g.L ? lo + g.chunk : g.L;
    int32_t* outp = p.out + static_cast<int64_t>(row) * k;
    uint2* region = kv_region(p, row);
    uint32_t* ctr = kvx_ctr(p, row);  // [0] committed slots, [1] frontier entries
    // Wave-private stage: commits from the bottom, frontier entries from the top.
    uint2* stg = sm.front + wave() * kWaveCap;
    uint32_t sc_n = 0, sq_n = 0;
    auto flush = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        uint32_t cb = 0, qb = 0;
        if (lane() == 0) {
            if (sc_n) cb = atomicAdd(&ctr[0], sc_n);
            if (sq_n) qb = atomicAdd(&ctr[1], sq_n);
        }
        cb = readlane(cb, 0);
        qb = readlane(qb, 0);
        for (uint32_t e = lane(); e < sc_n; e += 64) {
            const uint32_t slot = cb + e;
            if (slot < k) outp[slot] = static_cast<int32_t>(stg[e].x);
        }
        for (uint32_t e = lane(); e < sq_n; e += 64) region[qb + e] = stg[kWaveCap - 1 - e];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        sc_n = 0;
        sq_n = 0;
    };
    const Span sp = make_span(p.logits + static_cast<int64_t>(row) * p.stride, lo, hi);
    scan_span<kSegVec>(sp, NoPre{}, [&](u32x4 b, uint32_t i0) {
        bool pc[4], pq[4];
        uint64_t mc[4], mq[4];
        uint32_t tc = 0, tq = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool v = b[u] != kNoElem;
            const uint32_t c = coarse_of_bits(b[u]);
            pc[u] = v && c < tau;
            pq[u] = v && c == tau;
            mc[u] = __ballot(pc[u]);
            mq[u] = __ballot(pq[u]);
            tc += __builtin_popcountll(mc[u]);
            tq += __builtin_popcountll(mq[u]);
        }
        if (tc + tq == 0) return;
        if (sc_n + sq_n + tc + tq > static_cast<uint32_t>(kWaveCap)) flush();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (pc[u]) stg[mbcnt_from(mc[u], sc_n)] = make_uint2(i0 + u, 0u);
            sc_n += __builtin_popcountll(mc[u]);
            if (pq[u]) stg[kWaveCap - 1 - mbcnt_from(mq[u], sq_n)] = make_uint2(i0 + u, desc_key(b[u]));
            sq_n += __builtin_popcountll(mq[u]);
        }
    });
    flush();
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void kvx_finish_kernel(Params p) {
    __shared__ Shared sm;
    const uint32_t row = kvx_row();
    if (row >= static_cast<uint32_t>(p.m_cap)) return;
    const int32_t nvr = *p.num_valid_rows;
    const int32_t ke_row = p.ke[row];
    if (row >= clamp_len(nvr, p.m_cap)) return;
    const uint32_t k = p.k;
    if (clamp_len(ke_row, p.n) <= k) return;
    const uint32_t before = kv_counts(p, row)[1];
    uint32_t* ctr = kvx_ctr(p, row);
    const uint32_t nq = ctr[1];
    uint32_t* h0 = sm.hist[0];
    uint32_t* h1 = sm.hist[1];
    clear_hist(h1);
    if (threadIdx.x == 0) {
        sm.kext[0] = kNoElem;
        sm.kext[1] = 0;
    }
    __syncthreads();  // every thread has read the counters
    if (threadIdx.x == 0) {
        ctr[0] = 0;
        ctr[1] = 0;
    }
    count_route(p, TOPKF_ROUTE_EXACT_DIRECT);
    const uint32_t kq = k - before;
    int32_t* outp = p.out + static_cast<int64_t>(row) * k;
    uint2* region = kv_region(p, row);
    uint2* region2 = region + slice_len(p.n);
    if (nq <= static_cast<uint32_t>(kBlock * kRegs)) {
        refine_regs<kRegs>(
            [&](int u, uint32_t& i, uint32_t& key) {
                const uint32_t gi = threadIdx.x + kBlock * u;
                const bool on = gi < nq;
                const uint2 t2 = region[on ? gi : 0u];
                i = t2.x;
                key = t2.y;
                return on;
            },
            h1, h0, kq, before, outp, k, sm);
        return;
    }
    count_route(p, TOPKF_ROUTE_SPILL);
    // A large frontier whose keys are all equal (a constant row, say) needs
    // no refinement: any kq of its entries complete the output.
    uint32_t mn = kNoElem, mx = 0;
    for (uint32_t e = threadIdx.x; e < nq; e += kBlock) {
        const uint32_t key = region[e].y;
        mn = key < mn ? key : mn;
        mx = key > mx ? key : mx;
    }
    lds_extremes(&sm.kext[0], mn, mx);
    __syncthreads();
    if (sm.kext[0] == sm.kext[1]) {
        for (uint32_t j = threadIdx.x; j < kq; j += kBlock)
            outp[before + j] = static_cast<int32_t>(region[j].x);
        return;
    }
    for (uint32_t e = threadIdx.x; e < nq; e += kBlock) lds_inc(h1, region[e].y >> 21);
    if (threadIdx.x == 0) {
        sm.cnt[0] = nq;
        sm.out_cnt = before;
    }
    __syncthreads();
    const Frontier cur{sm.front, 0, region, &sm.cnt[0]};
    const Frontier nxt{sm.front, kFront, region2, &sm.cnt[1]};
    refine(cur, nxt, h1, h0, kq, outp, k, sm);
}

// Plain streaming read of nvec 16-byte vectors, the same 128-bit nontemporal
// loads as the selector's scan, four per thread in flight, folded into an
// XOR that is stored only if it equals an improbable value (so the loads
// cannot be dropped).  The bandwidth reference for the selector.
__global__ __launch_bounds__(kBlock) void read_probe_kernel(const u32x4* x, int64_t nvec, uint32_t* sink) {
    uint32_t acc = 0;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock * 4;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock * 4 + threadIdx.x; i < nvec; i += step) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + static_cast<int64_t>(u) * kBlock;
            v[u] = j < nvec ? __builtin_nontemporal_load(x + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

// One wave per coarse bin: the compile-time cutoff and the device search.
__global__ __launch_bounds__(kBlock) void cutoff_check_kernel(uint32_t* table, uint32_t* search) {
    const uint32_t tau = blockIdx.x * kWaves + wave();
    if (tau >= static_cast<uint32_t>(kBins)) return;
    const uint32_t c = wave_cutoff(tau);
    if (lane() == 0) {
        table[tau] = kCutoff.v[tau];
        search[tau] = c;
    }
}

__global__ void coarse_keys_kernel(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        out[i] = static_cast<uint16_t>(coarse_of_bits(__float_as_uint(x[i])));
}

// ------------------------------------------------------------------ host

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
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, persistent_kernel<128, true, false>, kBlock,
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
    if (pl.family == TOPKF_FAMILY_KVSPLIT && (pl.splits < 1 || pl.splits > kMaxSplits)) return false;
    if (pl.family == TOPKF_FAMILY_KVSPLIT && pl.min_segment < 4) return false;
    if (pl.primary_quarters < 4 || pl.primary_quarters > 31) return false;
    if (pl.dual && (pl.band_quarters <= pl.primary_quarters || pl.band_quarters > 32)) return false;
    return true;
}

topkf_status make_plan(int64_t m_cap, int64_t n, int32_t cus, int32_t occupancy,
                       topkf_plan* pl) {
    if (m_cap < 0 || n < 1 || cus < 1 || !pl) return TOPKF_EINVAL;
    if (occupancy < 1) occupancy = 1;
    topkf_plan r{};
    // View policy (Sec. 5.5: s = 64 and s = 128 compile-time policies;
    // Sec. 6.4 Fig. 12: sampling pays off for wide rows, exact localization
    // for short ones).  Measured on MI355X at K = 2048 over M = 64..4096
    // (ke ~ U[N/2, N]): the exact route keeps a row of up to 8K scores in
    // registers and wins below 8K columns, the two are within 5 % at 8K, and
    // past 8K (the exact route then reads the row twice) the view wins by
    // 25-40 % (10K: 11.5 / 15.9 us at M = 64, 89.9 / 119.9 us at M = 4096);
    // s = 128 is as fast as or faster than s = 64 (up to 12 % at 128K), so
    // s = 64 is left to explicit plans.
    r.stride = n <= 8192 ? 0 : 128;
    r.dual = r.stride ? 1 : 0;
    r.min_segment = 16384;
    // Secondary target K~1 = 2.5K (Sec. 4.6 treats K~ and K~1 as efficiency
    // knobs).  With the pages' 1.75K some causal-prefill rows (about 2 per
    // 1000) underfill both boundaries and recover through a whole-row exact
    // pass that holds their worker for the length of several rows; at 2.5K
    // the band rescues them in one extra read (measured: 8.6 % faster).
    r.band_quarters = 10;
    r.primary_quarters = 6;
    const int64_t pool = static_cast<int64_t>(cus) * occupancy;
    const int64_t rows = m_cap > 0 ? m_cap : 1;
    // Mapping (Sec. 5.5).  With at least a full pool of rows, persistent
    // workers.  With a quarter of the pool or fewer, one workgroup per row
    // unless the rows are long: KV-split pays for its second launch and its
    // replicated views from N >= 1024 * max(M, 64) columns (measured on
    // MI355X, ke ~ U[N/2, N], K = 2048, us per call, one workgroup per row
    // against the best split: 4 x 32K 13.0 / 15.2, 4 x 64K 18.3 / 15.9,
    // 64 x 64K 18.7 / 16.8, 128 x 64K 19.5 / 20.6, 128 x 128K 28.1 / 25.8,
    // 128 x 256K 42.8 / 36.3).  In between, KV-split: one workgroup per row
    // is up to 13 % faster on some i.i.d. shapes (256 x 128K: 32.1 / 36.4;
    // 384 x 128K: 52.9 / 51.0) but a row whose admitted tail is most of the
    // row (constant or heavily tied) then streams its whole frontier
    // through one workgroup, 3-4 times slower on the adversarial mix, where
    // the split spreads it over the parts.
    bool kv = false;
    if (r.stride != 0 && m_cap < pool) {
        if (4 * rows > pool) kv = true;
        else kv = n >= 1024 * (rows > 64 ? rows : 64);
    }
    if (!kv) {
        r.family = TOPKF_FAMILY_PERSISTENT;
        r.workers = static_cast<int32_t>(m_cap < pool ? rows : pool);
        r.splits = 1;
        // A worker that recovers an underfilled row re-reads it and holds up
        // the end of the launch.  On causal prefill (measured): K~ = 1.5K
        // (Sec. 4.2) rescues 2 % of rows with the band, 1.75K 0.2 %, 2K none
        // (Eq. 8 bound 0.02 %) at 30 % more candidates than 1.5K; the
        // candidates cost little since a row's refinement is one histogram
        // round, and 2K is 4 % faster than 1.75K (2.25K no faster).
        r.primary_quarters = 8;
    } else {
        // Parts per row: half the pool's slots over the rows (every part on
        // a CU of its own), at least 4 (at most 2 pool / M) so that the longest
        // rows of a ragged batch are split, and no segment shorter than 16K
        // columns (shorter segments lose more to the replicated view than
        // they gain in span).  Measured (us per call at 1 / 2 / 4 / 8 / 16
        // parts): 64 x 128K 34.0 / 25.0 / 20.6 / 21.4, 32 x 128K 33.5 / 24.5 /
        // 19.8 / 18.7, 128 x 128K 35.0 / 26.6 / 25.8 / 31.0, 64 x 512K 81.5 /
        // 52.0 / 38.1 / 41.0 / 46.1, 256 x 256K 60.8 / 58.8 / 58.6 / 61.6 /
        // 70.7; few long rows reach the segment floor first (4 x 512K: 32
        // parts 21.8 us).
        r.family = TOPKF_FAMILY_KVSPLIT;
        // Primary boundary only, at K~ = 2K.  Collecting the band in the
        // fused pass costs every part a second classification of every
        // score (decode: 31.7 us against 29.9 us), while at 2K the view
        // underfills rarely: the finite-population bound of Sec. 3.2 (Eq. 8)
        // puts it below 0.02 % of rows for s = 128 and L >= 32K, the order of
        // the residual exact-recovery rate the pages report for their
        // 1.5K/1.75K rescue policy (Sec. 6.4); an underfilled row still takes
        // the exact coarse route, so the result stays exact.
        r.dual = 0;
        r.primary_quarters = 8;
        // rounded down: a grid just above the CU count leaves some CUs two
        // parts and the launch waits for them (decode at 3 / 4 / 5 / 6 parts,
        // 192 / 256 / 320 / 384 workgroups: 22.2 / 20.4 / 24.4 / 23.9 us)
        const int64_t half_pool = pool / (2 * rows) > 1 ? pool / (2 * rows) : 1;
        const int64_t spread = (2 * pool + rows - 1) / rows;
        int64_t P = half_pool > (spread < 4 ? spread : 4) ? half_pool : (spread < 4 ? spread : 4);
        int64_t pmax = (n + r.min_segment - 1) / r.min_segment;
        if (pmax > kMaxSplits) pmax = kMaxSplits;
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
    if (pl.family == TOPKF_FAMILY_KVSPLIT && pl.stride == 0)
        *cb += static_cast<size_t>(m_cap) * kBins * sizeof(uint32_t);  // per-row coarse histograms
    const size_t per_owner = 2 * static_cast<size_t>(slice_len(n)) * sizeof(uint2);
    if (pl.family == TOPKF_FAMILY_PERSISTENT) {
        // two (index, key) slices per worker: wave spills, contiguous frontier
        *wb = static_cast<size_t>(pl.workers) * per_owner;
    } else {
        // per row: part ranges and contiguous frontier, then four words per part
        // (the two candidate counts and the smallest and largest stored key)
        *wb = static_cast<size_t>(m_cap) *
              (per_owner + 4 * static_cast<size_t>(pl.splits) * sizeof(uint32_t));
    }
}

template <int S, bool D, bool H>
hipError_t launch_family(const topkf_plan& pl, const Params& prm, hipStream_t st) {
    if (pl.family == TOPKF_FAMILY_PERSISTENT) {
        hipLaunchKernelGGL((persistent_kernel<S, D, H>), dim3(pl.workers), dim3(kBlock), 0, st, prm);
    } else {
        const int64_t total = static_cast<int64_t>(prm.m_cap) * pl.splits;
        const dim3 parts(static_cast<uint32_t>((total + 7) / 8 * 8));
        const dim3 rows(static_cast<uint32_t>((static_cast<int64_t>(prm.m_cap) + 7) / 8 * 8));
        if constexpr (S == 0) {
            // No view: the cooperative exact route.
            hipLaunchKernelGGL(kvx_hist_kernel, parts, dim3(kBlock), 0, st, prm);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kvx_cut_kernel, rows, dim3(kBlock), 0, st, prm);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kvx_classify_kernel, parts, dim3(kBlock), 0, st, prm);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kvx_finish_kernel, rows, dim3(kBlock), 0, st, prm);
        } else {
            hipLaunchKernelGGL((kvsplit_scan_kernel<S, D, H>), parts, dim3(kBlock), 0, st, prm);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((kvsplit_finish_kernel<S, D, H>), rows, dim3(kBlock), 0, st, prm);
        }
    }
    return hipGetLastError();
}

topkf_status run(const float* logits, int64_t m_cap, int64_t n, int64_t stride,
                 const int32_t* ke, int32_t* out, const int32_t* nvr, int32_t top_k,
                 void* counters, size_t counter_bytes, void* workspace, size_t workspace_bytes,
                 const topkf_plan* override_plan, const float* hint, uint32_t* stats,
                 hipStream_t st) {
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
    prm.band_q = pl.band_quarters;
    prm.prim_q = pl.primary_quarters;
    prm.hint = hint;
    // A proposal replaces the view's boundary; plans without a view take the
    // exact route whatever the proposal.
    const bool hinted = hint != nullptr && pl.stride != 0;
    hipError_t e;
    switch (pl.stride * 2 + pl.dual) {
        case 0: case 1: e = launch_family<0, false, false>(pl, prm, st); break;
        case 128: e = hinted ? launch_family<64, false, true>(pl, prm, st)
                             : launch_family<64, false, false>(pl, prm, st); break;
        case 129: e = hinted ? launch_family<64, true, true>(pl, prm, st)
                             : launch_family<64, true, false>(pl, prm, st); break;
        case 256: e = hinted ? launch_family<128, false, true>(pl, prm, st)
                             : launch_family<128, false, false>(pl, prm, st); break;
        default: e = hinted ? launch_family<128, true, true>(pl, prm, st)
                            : launch_family<128, true, false>(pl, prm, st); break;
    }
    return e == hipSuccess ? TOPKF_OK : TOPKF_EHIP;
}

// ------------------------------------------------------ allocation-free calls
//
// topk_filtered_noalloc takes its counters and workspace from one
// library-owned device array instead of caller buffers.  Every GPU the library
// runs on holds its own copy of the array until the process ends, and every
// call on that GPU shares it: calls that overlap on one GPU race.  Layout:
// the first kScratchCounterBytes are the counter buffer (zero between calls;
// cleared once per device, then returned to zero by every call), the rest is
// the workspace (any contents).
constexpr size_t kScratchBytes = static_cast<size_t>(256) << 20;
constexpr size_t kScratchCounterBytes = static_cast<size_t>(1) << 20;
constexpr size_t kScratchWorkBytes = kScratchBytes - kScratchCounterBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// A host-side handle of each device's copy of `scratch`: its device address
// (from hipGetSymbolAddress; the array's name in host code is no device
// address) and whether its counter part has been cleared.
struct ScratchRef {
    unsigned char* ptr = nullptr;
    bool cleared = false;
};
ScratchRef g_scratch[64];  // guarded by g_mu

__global__ __launch_bounds__(kBlock) void zero_words_kernel(uint4* p, int64_t n16) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * kBlock)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address; on the first call on a device the
// counter part is cleared on `st` (a fill kernel, so that a call captured in a
// HIP graph records no memset node).
topkf_status scratch_for_device(hipStream_t st, unsigned char** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TOPKF_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    ScratchRef& s = g_scratch[dev];
    if (!s.ptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TOPKF_EHIP;
        s.ptr = static_cast<unsigned char*>(ptr);
    }
    if (!s.cleared) {
        const int64_t n16 = static_cast<int64_t>(kScratchCounterBytes / 16);
        hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<uint32_t>(n16 / kBlock)), dim3(kBlock), 0,
                           st, reinterpret_cast<uint4*>(s.ptr), n16);
        if (hipGetLastError() != hipSuccess) return TOPKF_EHIP;
        // A clear recorded into a graph under capture has not run yet: clear
        // again on the next call.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) return TOPKF_EHIP;
        s.cleared = cs == hipStreamCaptureStatusNone;
    }
    *out = s.ptr;
    return TOPKF_OK;
}

// The automatic plan narrowed to the scratch: a plan whose workspace does not
// fit becomes the persistent mapping with as many workers as fit.
topkf_status noalloc_plan(int64_t m_cap, int64_t n, topkf_plan* pl) {
    DeviceInfo di;
    const topkf_status s = device_info(&di);
    if (s != TOPKF_OK) return s;
    make_plan(m_cap, n, di.cus, di.occupancy, pl);
    size_t cb = 0, wb = 0;
    plan_sizes(*pl, m_cap, n, &cb, &wb);
    if (cb > kScratchCounterBytes) return TOPKF_EWORKSPACE;
    if (wb <= kScratchWorkBytes) return TOPKF_OK;
    if (pl->family == TOPKF_FAMILY_KVSPLIT) {
        const int64_t pool = static_cast<int64_t>(di.cus) * di.occupancy;
        pl->family = TOPKF_FAMILY_PERSISTENT;
        pl->splits = 1;
        pl->dual = pl->stride ? 1 : 0;
        pl->primary_quarters = 7;
        pl->workers = static_cast<int32_t>(m_cap < pool ? m_cap : pool);
    }
    const size_t per_worker = 2 * static_cast<size_t>(slice_len(n)) * sizeof(uint2);
    const size_t fit = kScratchWorkBytes / per_worker;
    if (fit < 1) return TOPKF_EWORKSPACE;
    if (static_cast<size_t>(pl->workers) > fit) pl->workers = static_cast<int32_t>(fit);
    return TOPKF_OK;
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
               counter_bytes, workspace, workspace_bytes, nullptr, nullptr, nullptr, stream);
}

topkf_status topk_filtered_hinted(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                  int64_t row_stride, const int32_t* ke, int32_t* out,
                                  const int32_t* num_valid_rows, int32_t top_k, const float* hint,
                                  void* counters, size_t counter_bytes, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    if (num_rows > 0 && !hint) return TOPKF_EINVAL;
    return run(logits, num_rows, max_kv_len, row_stride, ke, out, num_valid_rows, top_k, counters,
               counter_bytes, workspace, workspace_bytes, nullptr, hint, nullptr, stream);
}

topkf_status topk_filtered_noalloc(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                   int64_t row_stride, const int32_t* ke, int32_t* out,
                                   const int32_t* num_valid_rows, int32_t top_k,
                                   hipStream_t stream) {
    if (num_rows < 0 || max_kv_len < 1 || row_stride < max_kv_len || top_k < 1 ||
        top_k > TOPKF_K_MAX)
        return TOPKF_EINVAL;
    if (max_kv_len > 0x7FFFFFFF || num_rows > 0x7FFFFFFF) return TOPKF_EUNSUPPORTED;
    if (num_rows == 0) return TOPKF_OK;
    if (!logits || !ke || !out || !num_valid_rows) return TOPKF_EINVAL;
    topkf_plan pl;
    topkf_status s = noalloc_plan(num_rows, max_kv_len, &pl);
    if (s != TOPKF_OK) return s;
    unsigned char* base = nullptr;
    s = scratch_for_device(stream, &base);
    if (s != TOPKF_OK) return s;
    return run(logits, num_rows, max_kv_len, row_stride, ke, out, num_valid_rows, top_k, base,
               kScratchCounterBytes, base + kScratchCounterBytes, kScratchWorkBytes, &pl, nullptr,
               nullptr, stream);
}

topkf_status topk_filtered_debug(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                 int64_t row_stride, const int32_t* ke, int32_t* out,
                                 const int32_t* num_valid_rows, int32_t top_k, void* counters,
                                 size_t counter_bytes, void* workspace, size_t workspace_bytes,
                                 const topkf_plan* plan, uint32_t* route_stats,
                                 hipStream_t stream) {
    return run(logits, num_rows, max_kv_len, row_stride, ke, out, num_valid_rows, top_k, counters,
               counter_bytes, workspace, workspace_bytes, plan, nullptr, route_stats, stream);
}

topkf_status topk_filtered_hinted_debug(const float* logits, int64_t num_rows,
                                        int64_t max_kv_len, int64_t row_stride, const int32_t* ke,
                                        int32_t* out, const int32_t* num_valid_rows, int32_t top_k,
                                        const float* hint, void* counters, size_t counter_bytes,
                                        void* workspace, size_t workspace_bytes,
                                        const topkf_plan* plan, uint32_t* route_stats,
                                        hipStream_t stream) {
    if (num_rows > 0 && !hint) return TOPKF_EINVAL;
    return run(logits, num_rows, max_kv_len, row_stride, ke, out, num_valid_rows, top_k, counters,
               counter_bytes, workspace, workspace_bytes, plan, hint, route_stats, stream);
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

topkf_status topkf_read_probe(const void* x, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (bytes < 0 || (bytes & 15)) return TOPKF_EINVAL;
    if (bytes == 0) return TOPKF_OK;
    if (!x || !sink || (reinterpret_cast<uintptr_t>(x) & 15)) return TOPKF_EINVAL;
    DeviceInfo di;
    const topkf_status st = device_info(&di);
    if (st != TOPKF_OK) return st;
    const int64_t nvec = bytes / 16;
    int64_t blocks = 2 * static_cast<int64_t>(di.cus);
    const int64_t need = (nvec + 4 * kBlock - 1) / (4 * kBlock);
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream,
                       static_cast<const u32x4*>(x), nvec, sink);
    return hipGetLastError() == hipSuccess ? TOPKF_OK : TOPKF_EHIP;
}

topkf_status topkf_coarse_cutoffs(uint32_t* table, uint32_t* search, hipStream_t stream) {
    if (!table || !search) return TOPKF_EINVAL;
    hipLaunchKernelGGL(cutoff_check_kernel, dim3(kBins / kWaves), dim3(kBlock), 0, stream, table, search);
    return hipGetLastError() == hipSuccess ? TOPKF_OK : TOPKF_EHIP;
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
