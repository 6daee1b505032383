// spec_verify.hip -- batched draft-verification sampler for gfx950 (MI355X).
//
// The method (what is computed) follows the speculative-decoding pages:
//   * greedy chain verification: accept the matching prefix of the K drafts
//     against the argmax of the target's verify rows, append the bonus
//     argmax (mini-sglang PR #134, "Modifications", verify_drafts);
//   * exact verification: accept draft j with probability min(1, p/q) in
//     order; at the first rejection sample normalize(relu(p - q)) and stop;
//     if all are accepted sample the last target row (spec-decode README,
//     "How it works" and "Provably exact");
//   * relaxed verification: accept iff p >= tau or the draft is in the
//     target top-k; mu = 1 on accepted drafts (nanospec README, acceptance
//     rules);
//   * greedy tree verification of an EAGLE-style draft tree (nanospec
//     README, intro and benchmark section).
//
// How it is computed here (no kernel design comes from the pages).  Every
// logit is read once, by streaming tiles: one workgroup of 256 threads
// reduces a 16 KB tile (8 KB for the greedy rule without log-probs) of one
// row to its max (with the lowest index among equal maxima for the greedy
// rules, and the rank count #{t : l_t > l_x} for the relaxed rule) and, where
// a normalizer is needed, the sum of exp(l - tile max): v_exp_f32 per logit,
// fp32 over a thread's terms, fp64 beyond.  Decisions and terminal draws are
// taken on the device in fp64, with a table-driven fp64 exp.
//
//   exact, relaxed, power: one launch (k_single).  Its first workgroups
//             stream the tiles in a grid-stride loop and publish each tile's
//             record; one sweep workgroup per (request, 2048- or 4096-token
//             chunk): the first R of a request (first in index order,
//             before every request's other sweep workgroups) each fold one
//             row's records and publish the row's record, then every one
//             reads the row records, decides, sums its chunk of the
//             terminal row(s) in fp64 and publishes the sums; the request's
//             last sweep workgroup draws the terminal token.
//
//   greedy: one launch (k_greedy): one workgroup per tile publishes the
//             tile's record, then one deciding workgroup per request folds
//             the records, tests the drafts and writes the outputs.
//
//   tree: one launch (k_tree): one workgroup per tile publishes the tile's
//             record, folding workgroups publish one record per row, and one
//             deciding workgroup per request reads the node rows' records,
//             runs the tests one lane per tree node and writes the outputs.
//
//   draft sampler: one launch (k_sample_rows): the tiles publish fp64 chunk
//             sums, and one workgroup per row draws.
//
//   vocabulary shards (spec_shard_*): k_stream per shard, then after the
//             caller's exchanges k_decide, or k_sweep and k_sample.
//
// Within a launch, workgroups hand data to each other through words in the
// workspace written and read with relaxed agent-scope atomics, which are
// coherent across the XCDs' L2 caches without a fence.  A published word is
// never zero, so zero means "not yet"; a waiting workgroup only waits on
// workgroups that start before it, and each wait is bounded.  Every
// reduction runs in a fixed order, so results are bitwise reproducible.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <limits.h>
#include <math.h>

#include <mutex>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileBytes = 16384;                        // streaming tile
constexpr int kTileVecs = kTileBytes / (kThreads * 16);  // 16-byte loads per thread
// The greedy rule's stream without log-probs reads bf16 rows in 8 KiB tiles:
// twice the workgroups, each with half the loads (measured: 8.68 vs 8.86 us
// for the [32][6][128256] target rows launched alone, 10.1 vs 10.4 us inside
// calls; the normalizer streams are no faster with them, and the tree's
// 61-row stream is slower, 23.8 vs 21.6 us).  A row then has as many tiles as
// an fp32 row of 16 KiB tiles.
constexpr int kSmallTileVecs = kTileVecs / 2;
constexpr int kStreamWavesPerSimd = 8;                   // k_stream occupancy target
constexpr int kChunk = 4096;                             // pass-2 tokens per workgroup
constexpr int kPass2WavesPerSimd = 4;                    // k_pass2 occupancy target
constexpr int kRun = kChunk / kThreads;                  // pass-2 tokens per thread
constexpr int kSweepGroups = 2;                          // pass-2 chunks per workgroup
constexpr int kSweepThreads = kThreads * kSweepGroups;   // k_sweep workgroup
constexpr int kSampleThreads = 1024;                     // k_sample workgroup
constexpr int kDecideThreads = 1024;                     // k_decide workgroup
constexpr int kSampleRun = kChunk / kSampleThreads;      // k_sample tokens per thread
constexpr int kSampleWaves = kSampleThreads / 64;
static_assert(kSampleRun == 4, "k_sample loads four tokens per thread");
constexpr int kMaxRows = 2 * SPEC_MAX_K + 1;
constexpr int kMaxB = SPEC_MAX_B;
// Tiles per row at SPEC_MAX_V (fp32 has the most): one record per lane.
constexpr int kMaxTiles = (SPEC_MAX_V * 4 + kTileBytes - 1) / kTileBytes;
static_assert(kMaxTiles <= 64, "a row's tile records must fit one wave");
constexpr int kMaxC2 = (SPEC_MAX_V + kChunk - 1) / kChunk;
static_assert(kMaxC2 <= 64, "a row's pass-2 chunks must fit one wave");

// Sub-chunks: a sweep workgroup publishes its chunk's masses per 1024-token
// sub-chunk, so the draw rescans 1024 tokens (four per thread) instead of a
// whole chunk.
constexpr int kSub = 1024;
constexpr int kSubs = kChunk / kSub;

// A sweep workgroup of the single launch sums PER * kSweepChunk tokens
// (PER = 1 or 2: half of a draw chunk or all of it) and publishes one
// record: S, Sq, dmin and its sub-chunks' two sums (sweep_words(PER) words:
// seven or eleven).  The drawer's lane l combines the kSweepSplit / PER
// records of draw chunk l.  Half-chunk sweeps give twice the workgroups, each
// with half the fp64 work, which shortens the slowest one while the chip
// holds them all at once.
constexpr int kSweepChunk = 2048;
constexpr int kSweepSplit = kChunk / kSweepChunk;
constexpr int kSweepSubs = kSweepChunk / kSub;
constexpr int sweep_words(int per) { return 3 + 2 * per * kSweepSubs; }
static_assert(kSweepSplit * kSweepChunk == kChunk && kSweepSubs * kSub == kSweepChunk, "whole sub-chunks");

enum Mode { kGreedy = 0, kExact = 1, kRelaxed = 2, kTree = 3, kPower = 4 };

// Rules that stream the draft rows and test p/q.
constexpr bool uses_draft(int mode) { return mode == kExact || mode == kPower; }

// Statistics of one tile: max m, then the lowest index of the max (greedy,
// tree) or the rank count (relaxed), and s = sum over the tile of
// 2^(l*log2e - fl(m*log2e)), i.e. sum exp(l - m) up to the rounding of the
// reference.
struct alignas(16) Seg {
    float m;
    int ic;
    double s;
};
static_assert(sizeof(Seg) == 16, "one 16-byte load per record");

// What the decide kernel hands to the sweep and sampling kernels for one
// request: the decision and the reference maxima of the terminal row(s).
struct alignas(16) Decision {
    int n;         // first rejection (K: all accepted)
    int residual;  // exact rule and n < K: sample relu(p_n - q_n)
    int pad0, pad1;
    double Mt, Md;  // maxima of target row n and draft row n
    double cls;     // p > q  <=>  (l - Mt) - (d - Md) > cls
    double rn;      // p_n(x_n) / q_n(x_n) of the rejected draft
};

// Fp64 sums of one pass-2 chunk: exp(l - Mt) and exp(d - Md) over the chunk,
// and over its tokens classified p > q with the streamed normalizers; dmin is
// the smallest distance of a token's (l - Mt) - (d - Md) from that
// classification threshold (+inf when nothing was classified), so the
// sampling kernel can tell whether the exact fp64 threshold would classify
// any token of the chunk otherwise.
struct alignas(16) ChunkSums {
    double sa, sb, pa, pb, dmin, pad;
};

struct Layout {
    size_t frec, fsums, frow;  // published tile, chunk and row records
    size_t total;
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The workspace of an unsharded call: [published tile records B*R*tpr, two
// words each][published chunk records: B*2*C2 sweep records of seven words
// or B*C2 of eleven, or the draft sampler's two words per chunk][published
// row records B*R, two words each].  It is zero when a call starts
// (zero-filled once by its owner) and every call leaves every byte it wrote
// zero again, whatever the rule or shape: the single-launch calls read zero
// as "not published yet".
inline Layout make_layout(int B, int R, int tpr, int C2) {
    Layout L;
    L.frec = 0;
    L.fsums = align_up(L.frec + (size_t)B * R * tpr * 16, 256);
    // the most any call publishes there: B * C2 * kSweepSplit sweep records of
    // sweep_words(1) words (at least B * C2 records of sweep_words(2), and the
    // draft sampler's two words per chunk)
    L.frow = align_up(L.fsums + (size_t)B * C2 * kSweepSplit * sweep_words(1) * 8, 256);
    L.total = align_up(L.frow + (size_t)B * R * 16, 256);
    return L;
}

// --------------------------------------------------------------- element IO
// Rows are read with buffer loads: the resource descriptor carries the row's
// size, so the hardware returns zeros past its end and no bounds branch sits
// between the loads; every thread issues all of its loads before it waits.
// Row sizes on the 16-byte path are multiples of 16 bytes, so a vector is
// either wholly inside the row or wholly past it.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;  // in global memory
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data format

template <typename T>
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const T* row, int V) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(row), (short)0, V * (int)sizeof(T),
                                             kRsrcWord3);
}

// Workgroup-uniform reads of inputs through the scalar cache (constant
// address space).  They are counted apart from the vector loads, so waiting
// for one does not wait for a tile in flight.  Only memory that no kernel of
// the call writes is read this way.
__device__ inline int32_t sload_i32(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}
__device__ inline float sload_f32(const float* p) {
    return *(const __attribute__((address_space(4))) float*)(uintptr_t)p;
}

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bit patterns
    static constexpr int kVec = 8;
    __device__ static inline float at(const uint16_t* p, size_t i) {
        return __uint_as_float((uint32_t)p[i] << 16);
    }
    // element i's bits: sword loads the aligned dword that holds it by a
    // scalar load (that dword lies in the same allocation: device
    // allocations are aligned far beyond 4 bytes), half picks the element;
    // from_bits widens it
    __device__ static inline uint32_t sword(const uint16_t* p, int i) {
        return *(const __attribute__((address_space(4))) uint32_t*)((uintptr_t)(p + i) & ~(uintptr_t)3);
    }
    __device__ static inline uint32_t half(const uint16_t* p, int i, uint32_t w) {
        return ((uintptr_t)(p + i) & 2) ? (w >> 16) : (w & 0xffffu);
    }
    __device__ static inline float from_bits(uint32_t w) { return __uint_as_float(w << 16); }
    // element i's bits by a vector buffer load: 0, with no memory access, at
    // or past the descriptor's size
    __device__ static inline uint32_t bbits(__amdgpu_buffer_rsrc_t r, int i) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, i * 2, 0, 0);
    }
    template <int AUX = 0>
    __device__ static inline u32x4 vraw(__amdgpu_buffer_rsrc_t r, int e) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, e * 2, 0, AUX);
    }
    // VEC elements from e on, one buffer load each, packed like a vector
    __device__ static inline u32x4 sgather(__amdgpu_buffer_rsrc_t r, int e) {
        u32x4 q;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            q[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (e + 2 * j) * 2, 0, 0) |
                   ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (e + 2 * j + 1) * 2, 0, 0) << 16);
        return q;
    }
    // element j of a packed vector
    __device__ static inline float get(const u32x4& q, int j) {
        return __uint_as_float((j & 1) ? (q[j >> 1] & 0xffff0000u) : (q[j >> 1] << 16));
    }
    // tokens e .. e+3 (e a multiple of 4), -inf at or past V
    __device__ static inline void load4(__amdgpu_buffer_rsrc_t r, int e, int V, bool vec, float (&v)[4]) {
        uint32_t w0, w1;
        if (vec) {
            const auto q = __builtin_amdgcn_raw_buffer_load_b64(r, e * 2, 0, 0);
            w0 = q[0];
            w1 = q[1];
        } else {
            w0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, e * 2, 0, 0) |
                 ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, e * 2 + 2, 0, 0) << 16);
            w1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, e * 2 + 4, 0, 0) |
                 ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, e * 2 + 6, 0, 0) << 16);
        }
        v[0] = __uint_as_float(w0 << 16);
        v[1] = __uint_as_float(w0 & 0xffff0000u);
        v[2] = __uint_as_float(w1 << 16);
        v[3] = __uint_as_float(w1 & 0xffff0000u);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e + j >= V) v[j] = -INFINITY;
    }
    // VEC elements from e on (indices clamped to V-1), one load each, packed
    // like a 16-byte vector load
    __device__ static inline u32x4 gather_clamped(const uint16_t* pp, int e, int V) {
        const __attribute__((address_space(1))) uint16_t* p = (const __attribute__((address_space(1))) uint16_t*)pp;
        u32x4 q;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            q[j] = (uint32_t)p[min(e + 2 * j, V - 1)] | ((uint32_t)p[min(e + 2 * j + 1, V - 1)] << 16);
        return q;
    }
    __device__ static inline void unpack(const u32x4 q, float* v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(q[j] << 16);
            v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
        }
    }
    // Sets the elements e + i >= V of a packed vector to -inf (bits 0xff80).
    __device__ static inline void mask_tail(u32x4& q, int e, int V) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = (e + 2 * j < V) ? (q[j] & 0xffffu) : 0xff80u;
            const uint32_t hi = (e + 2 * j + 1 < V) ? (q[j] & 0xffff0000u) : 0xff800000u;
            q[j] = lo | hi;
        }
    }
};

template <>
struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static inline float at(const float* p, size_t i) { return p[i]; }
    __device__ static inline uint32_t sword(const float* p, int i) {
        return *(const __attribute__((address_space(4))) uint32_t*)(uintptr_t)(p + i);
    }
    __device__ static inline uint32_t half(const float*, int, uint32_t w) { return w; }
    __device__ static inline float from_bits(uint32_t w) { return __uint_as_float(w); }
    __device__ static inline uint32_t bbits(__amdgpu_buffer_rsrc_t r, int i) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0);
    }
    template <int AUX = 0>
    __device__ static inline u32x4 vraw(__amdgpu_buffer_rsrc_t r, int e) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, AUX);
    }
    __device__ static inline u32x4 sgather(__amdgpu_buffer_rsrc_t r, int e) {
        u32x4 q;
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = __builtin_amdgcn_raw_buffer_load_b32(r, (e + j) * 4, 0, 0);
        return q;
    }
    __device__ static inline float get(const u32x4& q, int j) { return __uint_as_float(q[j]); }
    __device__ static inline void load4(__amdgpu_buffer_rsrc_t r, int e, int V, bool vec, float (&v)[4]) {
        if (vec) {
            const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(q[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (e + j) * 4, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e + j >= V) v[j] = -INFINITY;
    }
    __device__ static inline u32x4 gather_clamped(const float* pp, int e, int V) {
        const __attribute__((address_space(1))) float* p = (const __attribute__((address_space(1))) float*)pp;
        u32x4 q;
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = __float_as_uint(p[min(e + j, V - 1)]);
        return q;
    }
    __device__ static inline void unpack(const u32x4 q, float* v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(q[j]);
    }
    __device__ static inline void mask_tail(u32x4& q, int e, int V) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e + j >= V) q[j] = 0xff800000u;
    }
};

// Loads this thread's NV packed vectors of the chunk [c0, c1): vector k
// holds elements c0 + (k * kThreads + tid) * VEC + [0, VEC).  Elements at or
// past c1 read as -inf.  `vec` selects the 16-byte path (row start and size
// 16-byte aligned); otherwise each element is loaded on its own.  Values stay
// packed (bf16: two per register) until they are used.
// Thread tid (of kThreads) of the chunk [c0, c1): vector k covers tokens
// c0 + (k*kThreads + tid)*VEC + [0, VEC); tokens past c1 are masked.
template <typename T, int NV>
__device__ inline void load_chunk(__amdgpu_buffer_rsrc_t r, int c0, int c1, bool vec, int tid, u32x4 (&q)[NV]) {
    constexpr int VEC = Elem<T>::kVec;
    const int t0 = c0 + tid * VEC;
#pragma unroll
    for (int k = 0; k < NV; ++k)
        q[k] = vec ? Elem<T>::vraw(r, t0 + k * kThreads * VEC) : Elem<T>::sgather(r, t0 + k * kThreads * VEC);
    if (c1 - c0 < NV * kThreads * VEC) {  // partial chunk (uniform per workgroup)
#pragma unroll
        for (int k = 0; k < NV; ++k) Elem<T>::mask_tail(q[k], t0 + k * kThreads * VEC, c1);
    }
}

// Loads NV packed vectors of consecutive tokens [e0, e0 + NV*VEC) (one
// thread's contiguous run); tokens at or past V read as -inf.
template <typename T, int NV>
__device__ inline void load_run(__amdgpu_buffer_rsrc_t r, int e0, int V, bool vec, u32x4 (&q)[NV]) {
    constexpr int VEC = Elem<T>::kVec;
#pragma unroll
    for (int k = 0; k < NV; ++k) q[k] = vec ? Elem<T>::vraw(r, e0 + k * VEC) : Elem<T>::sgather(r, e0 + k * VEC);
#pragma unroll
    for (int k = 0; k < NV; ++k) Elem<T>::mask_tail(q[k], e0 + k * VEC, V);
}

// ------------------------------------------------------------ fp64 exp(x<=0)
// Reduction x = k ln2/512 + r with k = rint(x * 512/ln2) and |r| <= ln2/1024,
// a degree-3 Taylor polynomial (truncation error r^4/24 < 9e-15 relative)
// and 2^(k/512) = 2^(k>>9) * tab[k & 511], the power of two applied by
// v_ldexp.  k is rounded by adding 1.5 * 2^52 in the fma that scales x (the
// integer then sits in the low bits of the sum; one subtraction recovers it
// as a double).  r uses the double nearest ln2/512 in one fma: its error,
// |k| * 2^-63, stays below 3e-15 relative for x >= -30 and below 1e-13 at the
// clamp.  x is first clamped to -1000 (which also maps -inf to -1000), where
// v_ldexp underflows to exactly 0.  Branch-free; every op is full rate.
constexpr int kExpTab = 512;
constexpr double kInvLn2x512 = 0x1.71547652b82fep+9;  // 512 / ln 2
constexpr double kLn2o512 = 0x1.62e42fefa39efp-10;    // ln 2 / 512
constexpr double kRoundMagic = 0x1.8p52;              // 1.5 * 2^52

__device__ inline double exp_nonpos(double x, const double* tab) {
    const double xc = fmax(x, -1000.0);
    const double t = fma(xc, kInvLn2x512, kRoundMagic);  // 1.5 * 2^52 + k, |k| < 2^20
    const int k = (int)(uint32_t)__double_as_longlong(t);
    const double kd = t - kRoundMagic;
    const double r = fma(-kd, kLn2o512, xc);
    double p = fma(r, 1.0 / 6.0, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    return ldexp(tab[k & (kExpTab - 1)] * p, k >> 9);
}

// exp_nonpos of N values at once: the reductions and polynomials first, then
// all N table reads, then the scalings, so the reads are in flight together
// instead of one LDS round trip per value.  Bit-identical to exp_nonpos.
template <int N>
__device__ inline void exp_nonpos_n(const double (&x)[N], double (&e)[N], const double* tab) {
    double p[N], tv[N];
    int k[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const double xc = fmax(x[i], -1000.0);
        const double t = fma(xc, kInvLn2x512, kRoundMagic);
        k[i] = (int)(uint32_t)__double_as_longlong(t);
        const double kd = t - kRoundMagic;
        const double r = fma(-kd, kLn2o512, xc);
        double q = fma(r, 1.0 / 6.0, 0.5);
        q = fma(q, r, 1.0);
        p[i] = fma(q, r, 1.0);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) tv[i] = tab[k[i] & (kExpTab - 1)];
#pragma unroll
    for (int i = 0; i < N; ++i) e[i] = ldexp(tv[i] * p[i], k[i] >> 9);
}

// 1/k! as a double (k! is exact in binary64 for k <= 18)
constexpr double inv_factorial(int k) {
    double f = 1.0;
    for (int i = 2; i <= k; ++i) f *= i;
    return 1.0 / f;
}
constexpr double kLn2o16 = 0x1.62e42fefa39efp-5;  // ln 2 / 16
constexpr int kTabDegree = 15;

// The workgroup's table of 2^(j/512), j < 512, in LDS (the fp64 exp reads it
// per token), computed in place instead of loaded (a copy from memory cost a
// memory round trip at the start of every workgroup, all of them reading the
// same lines at once).  2^(j/512) = 2^(h/16) * 2^(l/512) with j = 32h + l:
// the first 48 threads take the 16 + 32 factors e^y, y = h ln2/16 or
// l ln2/512, by their Taylor series to degree 15 in Horner form (truncation
// below 1e-17 for y < ln 2), then every entry is one product.  Each entry is
// within 1.9 ulp of the exact value.  Called by every thread of the
// workgroup (it has a barrier); the caller's barrier publishes the table.
__device__ inline void fill_exp_table(double* tab) {
    __shared__ double fac[48];
    const int t = threadIdx.x;
    if (t < 48) {
        const double y = t < 16 ? (double)t * kLn2o16 : (double)(t - 16) * kLn2o512;
        double p = inv_factorial(kTabDegree);
#pragma unroll
        for (int k = kTabDegree - 1; k >= 0; --k) p = fma(p, y, inv_factorial(k));
        fac[t] = p;
    }
    __syncthreads();
    for (int j = t; j < kExpTab; j += blockDim.x) tab[j] = fac[j >> 5] * fac[16 + (j & 31)];
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;

// ------------------------------------------------------------ wave helpers
// Cross-lane steps use DPP (operands moved between lanes inside the VALU),
// not LDS permutes: reductions and scans are fixed sequences of lane moves,
// so every result is bit-reproducible.  Rows are 16 lanes, banks 4 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within a row
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr3 = 0x113, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142;  // lane 15 of each row -> next row
constexpr int kDppBcast31 = 0x143;  // lane 31 -> rows 2 and 3

// Lanes that are masked off, or whose source lane does not exist, receive
// `old`.
template <int CTRL, int RM = 0xF, int BM = 0xF>
__device__ inline int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, RM, BM, false);
}
template <int CTRL, int RM = 0xF, int BM = 0xF>
__device__ inline float dpp_f(float old, float v) {
    return __int_as_float(dpp_i<CTRL, RM, BM>(__float_as_int(old), __float_as_int(v)));
}
template <int CTRL, int RM = 0xF, int BM = 0xF>
__device__ inline double dpp_d(double old, double v) {
    const long long o = __double_as_longlong(old), u = __double_as_longlong(v);
    const int lo = dpp_i<CTRL, RM, BM>((int)o, (int)u);
    const int hi = dpp_i<CTRL, RM, BM>((int)(o >> 32), (int)(u >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ inline double readlane_d(double v, int l) {
    const long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)u, l);
    const int hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Wave total in every lane: butterfly within rows, then rows 1 and 3 pick up
// rows 0 and 2, then row 3 picks up rows 0-1; lane 63 holds the total.
__device__ inline double wave_sum(double v) {
    v += dpp_d<kDppXor1>(0.0, v);
    v += dpp_d<kDppXor2>(0.0, v);
    v += dpp_d<kDppHalfMirror>(0.0, v);
    v += dpp_d<kDppMirror>(0.0, v);
    v += dpp_d<kDppBcast15, 0xA>(0.0, v);
    v += dpp_d<kDppBcast31, 0xC>(0.0, v);
    return readlane_d(v, 63);
}

__device__ inline int wave_sum_i(int v) {
    v += dpp_i<kDppXor1>(0, v);
    v += dpp_i<kDppXor2>(0, v);
    v += dpp_i<kDppHalfMirror>(0, v);
    v += dpp_i<kDppMirror>(0, v);
    v += dpp_i<kDppBcast15, 0xA>(0, v);
    v += dpp_i<kDppBcast31, 0xC>(0, v);
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ inline void argmax_combine(float& m, int& idx, float om, int oi) {
    if (om > m || (om == m && oi < idx)) {
        m = om;
        idx = oi;
    }
}

template <int CTRL, int RM = 0xF>
__device__ inline void argmax_step(float& m, int& idx) {
    const float om = dpp_f<CTRL, RM>(m, m);  // masked-off lanes combine with themselves
    const int oi = dpp_i<CTRL, RM>(idx, idx);
    argmax_combine(m, idx, om, oi);
}

// Wave max with the lowest index among equal maxima, in every lane.
__device__ inline void wave_argmax(float& m, int& idx) {
    argmax_step<kDppXor1>(m, idx);
    argmax_step<kDppXor2>(m, idx);
    argmax_step<kDppHalfMirror>(m, idx);
    argmax_step<kDppMirror>(m, idx);
    argmax_step<kDppBcast15, 0xA>(m, idx);
    argmax_step<kDppBcast31, 0xC>(m, idx);
    m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
    idx = __builtin_amdgcn_readlane(idx, 63);
}

template <int CTRL, int RM = 0xF>
__device__ inline float max_step(float m) {
    return fmaxf(m, dpp_f<CTRL, RM>(m, m));
}

__device__ inline float wave_max(float m) {
    m = max_step<kDppXor1>(m);
    m = max_step<kDppXor2>(m);
    m = max_step<kDppHalfMirror>(m);
    m = max_step<kDppMirror>(m);
    m = max_step<kDppBcast15, 0xA>(m);
    m = max_step<kDppBcast31, 0xC>(m);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
}

// Inclusive prefix sum over the 64 lanes (in lane order).
__device__ inline double wave_incl_scan(double v) {
    double s = v + dpp_d<kDppShr1>(0.0, v);
    s += dpp_d<kDppShr2>(0.0, v);
    s += dpp_d<kDppShr3>(0.0, v);
    s += dpp_d<kDppShr4, 0xF, 0xE>(0.0, s);
    s += dpp_d<kDppShr8, 0xF, 0xC>(0.0, s);
    s += dpp_d<kDppBcast15, 0xA>(0.0, s);
    s += dpp_d<kDppBcast31, 0xC>(0.0, s);
    return s;
}

// Smallest double over the wave, in every lane.
__device__ inline double wave_min_d(double v) {
    v = fmin(v, dpp_d<kDppXor1>(v, v));
    v = fmin(v, dpp_d<kDppXor2>(v, v));
    v = fmin(v, dpp_d<kDppHalfMirror>(v, v));
    v = fmin(v, dpp_d<kDppMirror>(v, v));
    v = fmin(v, dpp_d<kDppBcast15, 0xA>(v, v));
    v = fmin(v, dpp_d<kDppBcast31, 0xC>(v, v));
    return readlane_d(v, 63);
}

// Smallest / largest int over the wave, in every lane.
__device__ inline int wave_min_i(int v) {
    v = min(v, dpp_i<kDppXor1>(v, v));
    v = min(v, dpp_i<kDppXor2>(v, v));
    v = min(v, dpp_i<kDppHalfMirror>(v, v));
    v = min(v, dpp_i<kDppMirror>(v, v));
    v = min(v, dpp_i<kDppBcast15, 0xA>(v, v));
    v = min(v, dpp_i<kDppBcast31, 0xC>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ inline int wave_max_i(int v) {
    v = max(v, dpp_i<kDppXor1>(v, v));
    v = max(v, dpp_i<kDppXor2>(v, v));
    v = max(v, dpp_i<kDppHalfMirror>(v, v));
    v = max(v, dpp_i<kDppMirror>(v, v));
    v = max(v, dpp_i<kDppBcast15, 0xA>(v, v));
    v = max(v, dpp_i<kDppBcast31, 0xC>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}

// ------------------------------------------------------------------- args
struct Args {
    const void* T;
    const void* D;
    const int32_t* tok;        // draft tokens [B][K] or node tokens [B][N]
    const int32_t* parents;    // [B][N] (tree)
    const int32_t* num_nodes;  // [B] or null (tree)
    const float* u;            // [B][K+1]
    int B, K, V;
    int rows_t;  // target rows per request: K+1, or N for a tree
    int R;       // rows streamed per request
    int tpr;     // streaming tiles per row
    int C2;      // pass-2 chunks per row
    int C2s;        // single launch: 2048-token sweep chunks per request
    int vec_t, vec_d;
    float tau;
    float alpha;  // power rule exponent
    int top_k;
    int32_t* out_tok;
    int32_t* out_len;
    float* out_tlp;
    float* out_blp;
    int32_t* out_status;
    int32_t* out_path;
    int L;  // output row length: K+1, or N for a tree
    unsigned char* ws;
    Seg* segs;        // [B][R][tpr]; sharded combine: G slots of these
    Decision* dec;    // [B]
    ChunkSums* sums;  // [B][C2]; sharded sample: G slots of these
    // vocabulary sharding (V above is then the shard's column count)
    int Vtot;              // vocabulary size: the bound of token ids
    int G, shard;          // shards, and the shard this call runs for
    size_t slot_segs;      // records between shard slots
    size_t slot_xv;        // floats between the slots' drafted-token logits
    const float* xv_in;    // gathered drafted-token logits, slot 0 ([B][K][2])
    float* xv_out;         // this shard's drafted-token logits ([B][K][2])
    size_t sums_slot;      // bytes between the shard slots of chunk sums
    int32_t* out_owner;    // [B] shard holding the terminal draw, or null
    // single-launch calls: published words
    uint64_t* frec;     // [B][R][tpr] tile records, two words each
    uint64_t* fsums;    // [B][sweep workgroups] sweep records (sweep_words words each)
    uint64_t* frow;     // [B][R] folded row records, two words each
    int nstream;        // workgroups of the launch that stream tiles
    int spin_limit;     // polling rounds of a wait before it gives up (status 2)
};

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <typename T>
__device__ inline const T* uniform_ptr(const T* p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = (uint32_t)uniform((int)(uint32_t)u), hi = (uint32_t)uniform((int)(uint32_t)(u >> 32));
    return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------- published words
// Single-launch calls pass tile records and chunk sums between workgroups of
// one launch, on any XCD, through 64-bit words written and read with
// agent-scope relaxed atomics (coherent across the XCDs' L2 caches without
// a fence).  A word of zero means "not written yet": every published word is
// encoded so it is never zero, the reader waits (a bounded spin) until every
// word it needs is non-zero, and the call's last workgroup for a request
// zeroes that request's words again.  The workspace region holding them must
// therefore be zero when a call starts; every call leaves it so.
__device__ inline uint64_t load_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_word(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr uint64_t kTop = 1ull << 63;
// A non-negative double (or NaN, or +inf) with its sign bit flipped: never
// zero, since none of them is -0.0.
__device__ inline uint64_t enc_nonneg(double v) { return (uint64_t)__double_as_longlong(v) ^ kTop; }
__device__ inline double dec_nonneg(uint64_t w) { return __longlong_as_double((long long)(w ^ kTop)); }
// Tile record {m, ic, s}: word 0 = valid bit | ic (31 bits, ic in [0, INT_MAX])
// | the bits of m; word 1 = s encoded as above (s >= 0 or NaN).
__device__ inline void publish_record(uint64_t* w, const Seg& sg) {
    store_word(w, kTop | ((uint64_t)((uint32_t)sg.ic & 0x7fffffffu) << 32) | __float_as_uint(sg.m));
    store_word(w + 1, enc_nonneg(sg.s));
}
__device__ inline Seg decode_record(uint64_t w0, uint64_t w1) {
    Seg sg;
    sg.m = __uint_as_float((uint32_t)w0);
    sg.ic = (int)((w0 >> 32) & 0x7fffffffu);
    sg.s = dec_nonneg(w1);
    return sg;
}
// The record of a tile with nothing in it (the fold's identity).
__device__ inline Seg neutral_record(bool argmax) {
    Seg sg;
    sg.m = -INFINITY;
    sg.ic = argmax ? INT_MAX : 0;
    sg.s = 0.0;
    return sg;
}
// Default bound of every wait for published words, in polling rounds (each
// round trip is about a microsecond, so about a second in all); a wait that
// runs out reports status 2 for its request instead of hanging the launch.
// Launches carry the bound in Args::spin_limit (spec_set_spin_limit).
constexpr int kSpinLimit = 1 << 20;

// Logit row g of the call (request g / R, row g % R of that request).  The
// result is wave-uniform, so loads use a scalar base and 32-bit offsets.
template <typename T, int MODE>
__device__ inline const T* call_row(const Args& a, int g, int& vec, int& active) {
    const int b = g / a.R, rr = g - (g / a.R) * a.R;
    active = 1;
    if (MODE == kTree && a.num_nodes) active = uniform(rr < min(max(a.num_nodes[b], 1), a.rows_t));
    if (uses_draft(MODE) && rr >= a.rows_t) {
        vec = a.vec_d;
        return uniform_ptr(reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + (rr - a.rows_t)) * a.V);
    }
    vec = a.vec_t;
    return uniform_ptr(reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + rr) * a.V);
}

// Issues this thread's loads of tile c of a row: vector k covers tokens
// c*TILE + (k*kThreads + tid)*VEC + [0, VEC).  Indices are clamped into the
// row and the caller masks tokens past V, so no load leaves the row.
template <typename T, bool NT, bool VECP, int NV>
__device__ inline void load_tile(const T* row, int V, int c, u32x4 (&q)[NV]) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int TILE = kThreads * NV * VEC;
    const int t0 = c * TILE + (int)threadIdx.x * VEC;
    if (VECP) {  // V is a multiple of VEC and every row is 16-byte aligned
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            // global (not flat) address space: these loads wait on vmcnt only
            const gu32x4* p = (const gu32x4*)(row + min(t0 + k * kThreads * VEC, V - VEC));
            q[k] = NT ? __builtin_nontemporal_load(p) : *p;
        }
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) q[k] = Elem<T>::gather_clamped(row, t0 + k * kThreads * VEC, V);
    }
}

// ----------------------------------------------------------- streaming pass
// Every logit row is read once, one tile per workgroup.  Per element: widen,
// max (or argmax, or rank compare), and for the normalizer one fma, one exp2
// and one add against the tile max, which the workgroup agrees on first.
// VECP: every row of the call takes the 16-byte path (chosen on the host).
// XV: the first workgroups (dispatched first, so the extra latency hides
// behind the rest of the grid) also record the drafted tokens' target and
// draft logits, one (request, position, row kind) each, for the decision
// kernels to load beside the tile records.  On a vocabulary shard only the
// shard whose columns hold the token records it.
// SHARD (a vocabulary shard's relaxed-rule statistics): the rank count's
// threshold l_x comes from the gathered drafted-token logits, since the token
// may be another shard's column.
// PUBLISH (the single-launch calls): the tile record goes out as two
// agent-scope atomic words (publish_record), which workgroups on any XCD of
// the same launch read coherently; otherwise it is a plain store that the
// next kernel reads.  blk is the tile's index in the call's streaming grid.
template <typename T, int MODE, bool SUM, bool VECP, bool XV, bool SHARD, int NV, bool PUBLISH>
__device__ __forceinline__ void stream_tile(const Args& a, const unsigned blk) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int TILE = kThreads * NV * VEC;
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    constexpr bool COUNT = (MODE == kRelaxed);
    // Non-temporal loads: the stream touches every line once.  (The one or
    // two rows the terminal sample re-reads are a small share, and measured
    // calls are faster this way.)
    constexpr bool NT = true;

    const int lane = threadIdx.x & 63;
    const int wave = uniform((int)(threadIdx.x >> 6));  // scalar: per-wave LDS addresses stay in SGPRs
    __shared__ float s_m[kWaves];
    __shared__ int s_j[kWaves];
    __shared__ double s_s[kWaves];

    // Waves issuing their loads take precedence over waves reducing a tile
    // that has arrived, so the memory system sees every load as early as
    // possible (measured: 0.4 us of 16 at the exact rule's B=32, K=5 shape).
    __builtin_amdgcn_s_setprio(3);
    const int g = uniform((int)(blk / (unsigned)a.tpr));
    const int c = (int)blk - g * a.tpr;
    int vec, act;
    const T* row = call_row<T, MODE>(a, g, vec, act);
    if (!act) return;  // tree node past num_nodes: never read
    // Drafted-token reads.  The token ids are workgroup-uniform scalar loads
    // issued right behind the tile's loads (their waits count apart from the
    // tile's vector loads, and nothing delays the tile's issue).
    // XV: the first workgroups record the drafted token's logits, one
    // (position, row kind) each: 2*B*K <= B*(2K+1) workgroups for the draft
    // rules, B*K <= B*(K+1) for the others.  The logit is a vector load issued
    // right behind the tile's and consumed only when the record is written, so
    // nothing waits for it; every workgroup issues it, with a descriptor of
    // size 0 (no memory access) outside the recording workgroups and for an
    // out-of-range token.
    constexpr int kinds = uses_draft(MODE) ? 2 : 1;
    const bool xvw = XV && (int)blk < kinds * a.B * a.K;
    const int xi = uniform((int)blk / kinds), xslot = 2 * xi + ((int)blk - xi * kinds);
    // COUNT: a target row j < K counts the tokens strictly above l_x of its
    // drafted token x; l_x is needed from the second pass over the tile on
    const int cb = COUNT ? g / a.R : 0, cr = COUNT ? g - cb * a.R : 0;
    const bool cw = COUNT && cr < a.K;
    u32x4 q[NV];
    load_tile<T, NT, VECP, NV>(row, a.V, c, q);
    __builtin_amdgcn_sched_barrier(0);
    int xt = 0, ct = 0;
    if (xvw) xt = sload_i32(a.tok + xi);
    if (cw) ct = sload_i32(a.tok + cb * a.K + cr);
    uint32_t xraw = 0u;
    int xl = -1;
    if (XV) {
        const int b = xi / a.K, j = xi - b * a.K;
        const T* xsrc = xslot & 1 ? reinterpret_cast<const T*>(a.D) + (size_t)xi * a.V
                                  : reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + j) * a.V;
        xl = xvw ? xt - a.shard * a.V : -1;
        const bool xin = (unsigned)xl < (unsigned)a.V;
        xraw = Elem<T>::bbits(row_rsrc(uniform_ptr(xsrc), xin ? a.V : 0), xin ? xl : 0);
    }
    // relaxed: the raw word holding l_x, turned into the threshold after the
    // first barrier (so that its wait falls there)
    uint32_t tword = 0u;
    const bool tin = cw && (SHARD ? (unsigned)ct < (unsigned)a.Vtot : (unsigned)ct < (unsigned)a.V);
    if (tin) {
        if (SHARD)
            tword = (uint32_t)__float_as_uint(sload_f32(a.xv_in + (size_t)(ct / a.V) * a.slot_xv + cb * a.K + cr));
        else
            tword = Elem<T>::sword(row, ct);
    }
    __builtin_amdgcn_s_setprio(0);

    const int t0 = c * TILE + (int)threadIdx.x * VEC;
    if (c == a.tpr - 1 && a.V % TILE != 0) {  // ragged last tile: clamped lanes
#pragma unroll
        for (int k = 0; k < NV; ++k) Elem<T>::mask_tail(q[k], t0 + k * kThreads * VEC, a.V);
    }
    // Values are unpacked from the packed vectors where they are used, so
    // only the 16-byte vectors stay live between the phases.
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float v[VEC];
        Elem<T>::unpack(q[k], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) m = fmaxf(m, v[i]);
    }
    float M = wave_max(m);
    if (lane == 0) s_m[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    int I = 0;
    // relaxed: count the tokens strictly above l_x
    const float thr = !tin ? INFINITY : SHARD ? __uint_as_float(tword) : Elem<T>::from_bits(Elem<T>::half(row, ct, tword));
    // Greedy rules: the lowest index holding the tile max.  Only threads whose
    // own max is the tile max search their tokens (ascending, first hit), so
    // the common path pays one max per token.
    int idx = INT_MAX;
    if (ARGMAX && m == M && M > -INFINITY) {
#pragma unroll
        for (int k = NV - 1; k >= 0; --k) {
            float v[VEC];
            Elem<T>::unpack(q[k], v);
#pragma unroll
            for (int i = VEC - 1; i >= 0; --i)
                if (v[i] == M) idx = t0 + k * kThreads * VEC + i;
        }
    }
    double s = 0.0;
    int cnt = 0;
    if (COUNT && !SUM) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            float v[VEC];
            Elem<T>::unpack(q[k], v);
#pragma unroll
            for (int i = 0; i < VEC; ++i) cnt += (v[i] > thr) ? 1 : 0;
        }
    }
    if (SUM && M > -INFINITY) {
        // 2^(l*L - mL) with the reference mL = fl(M*L): every term <= 1.  A
        // thread's 32 (bf16) or 16 (fp32) terms are summed in fp32 (relative
        // error below 2e-6 even in the worst case, about 4e-8 measured on
        // 3*N(0,1) tiles), then in fp64 across lanes and waves.
        const float mL = M * kLog2e;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            float v[VEC];
            Elem<T>::unpack(q[k], v);
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                acc += __builtin_amdgcn_exp2f(fmaf(v[i], kLog2e, -mL));
                if (COUNT) cnt += (v[i] > thr) ? 1 : 0;
            }
        }
        s = (double)acc;
    }
    if (SUM || ARGMAX || COUNT) {
        if (SUM) s = wave_sum(s);
        if (ARGMAX) idx = wave_min_i(idx);
        if (COUNT) cnt = wave_sum_i(cnt);
        if (lane == 0) {
            s_s[wave] = s;
            s_j[wave] = ARGMAX ? idx : cnt;
        }
        __syncthreads();
        s = ((s_s[0] + s_s[1]) + s_s[2]) + s_s[3];
        if (ARGMAX) I = min(min(s_j[0], s_j[1]), min(s_j[2], s_j[3]));
        if (COUNT) I = ((s_j[0] + s_j[1]) + s_j[2]) + s_j[3];
    }
    if (threadIdx.x == 0) {
        Seg sg;
        sg.m = M;
        sg.ic = (ARGMAX || COUNT) ? I : 0;
        sg.s = s;
        if (PUBLISH)
            publish_record(a.frec + 2 * (size_t)blk, sg);
        else
            a.segs[blk] = sg;
        if (xvw && (unsigned)xl < (unsigned)a.V) a.xv_out[xslot] = Elem<T>::from_bits(xraw);
    }
}

template <typename T, int MODE, bool SUM, bool VECP, bool XV, bool SHARD, int NV>
__global__ __launch_bounds__(kThreads, kStreamWavesPerSimd) void k_stream(const Args a) {
    stream_tile<T, MODE, SUM, VECP, XV, SHARD, NV, false>(a, blockIdx.x);
}

// ------------------------------------------------------ sampler stream
// The draft sampler draws from every row it streams, so the fp64 chunk sums
// its inverse CDF needs are taken in the one pass: one workgroup per 16 KiB
// tile finds the tile max M, then sums exp(l - M) in fp64 (the table exp
// above) over each 4096-token chunk of the tile.  Each chunk's record is
// {sum, M}, published for the row's drawing workgroup, which rescales them to
// the row max.  One fp64 exp
// per token makes the pass VALU-bound, so it keeps eight waves per SIMD and
// takes the exps four at a time, their table reads in flight together.
constexpr int kRowWords = 2;  // published words per chunk of a sampled row

template <typename T, bool VECP>
__device__ __forceinline__ void rows_tile(const Args& a, const unsigned blk) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int TILE = kThreads * kTileVecs * VEC;
    constexpr int CPT = TILE / kChunk;  // chunks per tile: 2 (bf16) or 1 (fp32)
    static_assert(CPT * kChunk == TILE && kTileVecs % CPT == 0, "a tile holds whole chunks");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    __shared__ double tab[kExpTab];
    __shared__ float s_m[kWaves];
    __shared__ double s_s[kWaves][CPT];

    const int g = uniform((int)(blk / (unsigned)a.tpr));
    const int c = (int)blk - g * a.tpr;
    int vec, act;
    const T* row = call_row<T, kRelaxed>(a, g, vec, act);
    u32x4 q[kTileVecs];
    load_tile<T, true, VECP, kTileVecs>(row, a.V, c, q);
    fill_exp_table(tab);  // while the tile's loads are in flight
    const int t0 = c * TILE + (int)threadIdx.x * VEC;
    if (c == a.tpr - 1 && a.V % TILE != 0) {
#pragma unroll
        for (int k = 0; k < kTileVecs; ++k) Elem<T>::mask_tail(q[k], t0 + k * kThreads * VEC, a.V);
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kTileVecs; ++k) {
        float v[VEC];
        Elem<T>::unpack(q[k], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    if (lane == 0) s_m[wave] = m;
    __syncthreads();  // also publishes the exp table
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    // vector k of a thread lies in chunk k / (kTileVecs / CPT) of the tile
    double acc[CPT];
#pragma unroll
    for (int h = 0; h < CPT; ++h) acc[h] = 0.0;
    if (M > -INFINITY) {
#pragma unroll
        for (int k = 0; k < kTileVecs; ++k) {
            float v[VEC];
            Elem<T>::unpack(q[k], v);
#pragma unroll
            for (int i0 = 0; i0 < VEC; i0 += 4) {
                double x[4], e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (double)v[i0 + i] - (double)M;
                exp_nonpos_n<4>(x, e, tab);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[k / (kTileVecs / CPT)] += e[i];
            }
        }
    }
#pragma unroll
    for (int h = 0; h < CPT; ++h) {
        acc[h] = wave_sum(acc[h]);
        if (lane == 0) s_s[wave][h] = acc[h];
    }
    __syncthreads();
    if ((int)threadIdx.x < CPT) {
        const int h = threadIdx.x, ch = c * CPT + h;
        if (ch < a.C2) {
            // published as two never-zero words: the sum (>= +0) and the tile max
            uint64_t* w = a.fsums + ((size_t)g * a.C2 + ch) * kRowWords;
            store_word(w, enc_nonneg(((s_s[0][h] + s_s[1][h]) + s_s[2][h]) + s_s[3][h]));
            store_word(w + 1, kTop | (uint64_t)__float_as_uint(M));
        }
    }
}

// ------------------------------------------- drafted-token logits (shards)
// Step 0 of a sharded relaxed call: the logit of each drafted token in its
// target row, written by the shard whose columns hold the token.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_values(const Args a, float* out) {
    const int i = (int)(blockIdx.x * kThreads + threadIdx.x);
    if (i >= a.B * a.K) return;
    const int b = i / a.K, j = i - b * a.K;
    const int xl = a.tok[i] - a.shard * a.V;
    if ((unsigned)xl < (unsigned)a.V)
        out[i] = Elem<T>::at(reinterpret_cast<const T*>(a.T), (size_t)(b * a.rows_t + j) * a.V + xl);
}

// ------------------------------------------------------- read ceiling
// The streaming kernel's memory access with no arithmetic: one workgroup per
// 16 KiB tile, four non-temporal 16-byte loads per thread, an xor of the
// words so the loads stay live, one word written per workgroup.  Its rate is
// the practical ceiling the streaming kernel is measured against.
__global__ __launch_bounds__(kThreads, kStreamWavesPerSimd) void k_read(const unsigned char* data, size_t nvec,
                                                                      uint32_t* out) {
    const size_t v0 = (size_t)blockIdx.x * (kThreads * kTileVecs) + threadIdx.x;
    u32x4 q[kTileVecs];
#pragma unroll
    for (int k = 0; k < kTileVecs; ++k) {
        const size_t v = min(v0 + (size_t)k * kThreads, nvec - 1);
        q[k] = __builtin_nontemporal_load((const gu32x4*)(data + v * 16));
    }
    uint32_t x = 0u;
#pragma unroll
    for (int k = 0; k < kTileVecs; ++k) x ^= q[k].x ^ q[k].y ^ q[k].z ^ q[k].w;
    x = (uint32_t)wave_max_i((int)(x & 0x7fffffffu));
    __shared__ uint32_t s_x[kWaves];
    if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

// ------------------------------------------------------- row statistics
// Row max M, argmax g (lowest index), rank count c and log normalizer
// lnS = log sum exp(l - M) of the rows of one request, in LDS.
struct RowStats {
    float M[kMaxRows];
    int g[kMaxRows];
    int c[kMaxRows];
    double lnS[kMaxRows];
};

// Folds the tile records of rows [0, nrows) of request b into RowStats.
// Wave w of NW takes rows w, w + NW, ... in batches of kFoldBatch, one tile
// record per lane; load(k0, sg) fills the batch starting at k0 (neutral
// records for absent rows and lanes), and runs at least once in every wave.
// Ends with a barrier.
constexpr int kFoldBatch = 4;
template <int MODE, bool SUM, int NW, typename Load>
__device__ void fold_batches(int nrows, RowStats& rs, const double* tab, Load load) {
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    constexpr bool COUNT = (MODE == kRelaxed);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int k0 = 0; k0 == 0 || wave + NW * k0 < nrows; k0 += kFoldBatch) {
        Seg sg[kFoldBatch];
        load(k0, sg);
        double Sl = 1.0;  // lane j: normalizer of batch row j
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j) {
            const int r = wave + NW * (k0 + j);
            if (r >= nrows) break;
            float M = sg[j].m;
            int ic = sg[j].ic;
            if (ARGMAX)
                wave_argmax(M, ic);
            else
                M = wave_max(M);
            if (COUNT) ic = wave_sum_i(ic);
            if (SUM) {
                // tile sum * 2^(fl(m*L) - M*L), exact reference difference in fp64
                double t = 0.0;
                if (sg[j].m > -INFINITY) {
                    const float mL = sg[j].m * kLog2e;
                    t = sg[j].s * exp_nonpos(((double)mL - (double)M * (double)kLog2e) * kLn2, tab);
                }
                const double S = wave_sum(t);
                if (lane == j) Sl = S;
            }
            if (lane == 0) {
                rs.M[r] = M;
                rs.g[r] = ARGMAX ? ic : 0;
                rs.c[r] = COUNT ? ic : 0;
            }
        }
        if (SUM) {
            const double lS = log(Sl);  // one log for the whole batch
            const int r = wave + NW * (k0 + lane);
            if (lane < kFoldBatch && r < nrows) rs.lnS[r] = lS;
        }
    }
    __syncthreads();
}

// Records written by a previous kernel.  Every batch's loads are issued
// before any is used, and `hook` runs once in every thread after the first
// batch is issued, before any record is used: the caller's own loads go
// there, and the barrier that publishes the exp_nonpos table, so that all of
// them share one memory round trip.
template <int MODE, bool SUM, int NW, bool SHARD, typename Hook>
__device__ void fold_rows(const Args& a, int b, int nrows, RowStats& rs, const double* tab, Hook hook) {
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Sharded: lane l takes tile l % tpr of shard l / tpr's slot; a shard's
    // argmax is a column of its own, offset to a vocabulary index here.
    size_t off = lane;
    unsigned goff = 0u;
    int nrec = a.tpr;
    if (SHARD) {
        const int sl = lane / a.tpr;
        off = (size_t)sl * a.slot_segs + (lane - sl * a.tpr);
        goff = (unsigned)sl * (unsigned)a.V;
        nrec = a.G * a.tpr;
    }
    bool hooked = false;
    fold_batches<MODE, SUM, NW>(nrows, rs, tab, [&](int k0, Seg (&sg)[kFoldBatch]) {
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j) {
            const int r = wave + NW * (k0 + j);
            if (r < nrows && lane < nrec) {
                sg[j] = a.segs[((size_t)b * a.R + r) * a.tpr + off];
                if (SHARD && ARGMAX && sg[j].ic != INT_MAX) sg[j].ic = (int)((unsigned)sg[j].ic + goff);
            } else {
                sg[j] = neutral_record(ARGMAX);
            }
        }
        if (!hooked) {
            hook();
            hooked = true;
        }
    });
}

// Records published by the streaming workgroups of the same launch: each
// batch waits until its records' words are all written.  Returns false in a
// thread whose wait ran out (Args::spin_limit).
template <int MODE, bool SUM, int NW>
__device__ bool fold_rows_published(const Args& a, int b, int nrows, RowStats& rs, const double* tab) {
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bool ok = true;
    fold_batches<MODE, SUM, NW>(nrows, rs, tab, [&](int k0, Seg (&sg)[kFoldBatch]) {
        uint64_t w0[kFoldBatch], w1[kFoldBatch];
        const uint64_t* src[kFoldBatch];
        bool need[kFoldBatch];
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j) {
            const int r = wave + NW * (k0 + j);
            need[j] = r < nrows && lane < a.tpr;
            // a batch row past the last reads the last row's record and ignores it
            src[j] = a.frec + 2 * (((size_t)b * a.R + min(r, nrows - 1)) * a.tpr + lane);
            w0[j] = w1[j] = 0ull;
        }
        for (int it = 0;; ++it) {
            // lanes past the row's tiles read nothing; the others read every
            // word each round, so the loads of a round are in flight together
            if (lane < a.tpr) {
#pragma unroll
                for (int j = 0; j < kFoldBatch; ++j) {
                    w0[j] = load_word(src[j]);
                    w1[j] = load_word(src[j] + 1);
                }
            }
            bool missing = false;
#pragma unroll
            for (int j = 0; j < kFoldBatch; ++j) missing |= need[j] && (w0[j] == 0ull || w1[j] == 0ull);
            if (__ballot(missing) == 0ull) break;
            if (it >= a.spin_limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j)
            sg[j] = need[j] ? decode_record(w0[j], w1[j]) : neutral_record(ARGMAX);
    });
    return ok;
}

// ------------------------------------------------------ chain decision
// Per-draft inputs, held by lane j < K of wave 0.
struct ChainVals {
    int x;
    bool bad;
    float lx, dx, u;
};

// Draft token (and its uniform); issued before the row records are folded.
template <int MODE>
__device__ inline void chain_load_tokens(const Args& a, int b, ChainVals& cv) {
    const int j = threadIdx.x;
    cv.x = -1;
    cv.bad = false;
    cv.lx = cv.dx = -INFINITY;
    cv.u = 0.f;
    if (j < a.K) {
        cv.x = a.tok[b * a.K + j];
        if (uses_draft(MODE)) cv.u = a.u[b * (a.K + 1) + j];
    }
}

// Logits of the drafted token in target row j (and draft row j): depends on
// the token load, so it runs as the fold's hook.
// The streaming kernel recorded both logits (XV); on vocabulary shards, in
// the slot of the shard whose columns hold the token.  Unsharded, the load
// does not depend on the token, so it overlaps the record loads.
template <typename T, int MODE, bool SHARD>
__device__ inline void chain_load_values(const Args& a, int b, ChainVals& cv) {
    const int j = threadIdx.x;
    if (j < a.K) {
        cv.bad = (unsigned)cv.x >= (unsigned)a.Vtot;
        if (MODE == kGreedy) return;
        const float* xv = a.xv_in + 2 * (b * a.K + j);
        if (SHARD) {
            if (cv.bad) return;
            xv += (size_t)(cv.x / a.V) * a.slot_xv;
        }
        // unsharded: loaded whatever the token (a malformed token's entry is
        // stale and unused), so the load need not wait for it
        const float lx = xv[0];
        const float dx = uses_draft(MODE) ? xv[1] : -INFINITY;
        if (!cv.bad) {
            cv.lx = lx;
            cv.dx = dx;
        }
    }
}

struct ChainDecision {
    int n, bad_n;
    int x[64];
    double lp[64], lq[64], r[64], la[64];  // la: log acceptance probability (power)
};

// Wave 0: lane j < K evaluates the test of draft j in fp64; a ballot finds
// the first rejection n (lane K never accepts, so n <= K).  Results go to LDS.
template <int MODE>
__device__ void chain_decide(const Args& a, const RowStats& rs, const ChainVals& cv, ChainDecision& cd) {
    const int j = threadIdx.x, K = a.K;
    bool acc = false;
    double lp = 0.0, lq = 0.0, r = 0.0, la = -INFINITY;  // a malformed token is rejected outright
    if (j < K && !cv.bad) {
        if (MODE == kGreedy) {
            acc = (cv.x == rs.g[j]);
            lp = -rs.lnS[j];  // the accepted token is the row max
        } else {
            lp = ((double)cv.lx - (double)rs.M[j]) - rs.lnS[j];
            if (MODE == kExact) {
                lq = ((double)cv.dx - (double)rs.M[a.rows_t + j]) - rs.lnS[a.rows_t + j];
                if (lp == -INFINITY)
                    r = 0.0;
                else if (lq == -INFINITY)
                    r = INFINITY;
                else
                    r = exp(lp - lq);
                acc = (double)cv.u < r;
            } else if (MODE == kPower) {
                // accept with probability a = min(1, p/q)^alpha (alpha = 0:
                // always); r holds a, la its log
                lq = ((double)cv.dx - (double)rs.M[a.rows_t + j]) - rs.lnS[a.rows_t + j];
                const double al = (double)a.alpha;
                if (al == 0.0 || (lq == -INFINITY && lp > -INFINITY))
                    la = 0.0;
                else if (lp == -INFINITY)
                    la = -INFINITY;
                else
                    la = fmin(0.0, al * (lp - lq));
                r = exp(la);
                acc = (double)cv.u < r;
            } else {
                acc = (rs.c[j] < a.top_k) || (exp(lp) >= (double)a.tau);
            }
        }
    }
    const unsigned long long mask = __ballot(acc);
    const int n = __builtin_ctzll(~mask);
    cd.x[j] = cv.x;
    cd.lp[j] = lp;
    cd.lq[j] = lq;
    cd.r[j] = r;
    cd.la[j] = la;
    if (j == n) {
        cd.n = n;
        cd.bad_n = (n < K && cv.bad) ? 1 : 0;
    }
}

// Writes positions j < n (accepted drafts) and n < j < L (padding) of the
// chain outputs, plus accept_len and (with status) status.  Position n is the
// caller's.
template <int MODE>
__device__ void write_prefix(const Args& a, int b, const ChainDecision& cd, bool status = true) {
    const int n = cd.n, L = a.L;
    int32_t* otok = a.out_tok + (size_t)b * L;
    float* otlp = a.out_tlp ? a.out_tlp + (size_t)b * L : nullptr;
    float* oblp = a.out_blp ? a.out_blp + (size_t)b * L : nullptr;
    for (int j = threadIdx.x; j < L; j += blockDim.x) {
        if (j < n) {
            otok[j] = cd.x[j];
            if (otlp) otlp[j] = (float)cd.lp[j];
            if (oblp)
                oblp[j] = (MODE == kExact) ? (float)fmin(0.0, cd.lp[j] - cd.lq[j])
                                           : (MODE == kPower ? (float)cd.la[j] : 0.f);
        } else if (j > n) {
            otok[j] = -1;
            if (otlp) otlp[j] = 0.f;
            if (oblp) oblp[j] = 0.f;
        }
    }
    if (threadIdx.x == 0) {
        a.out_len[b] = n;
        if (status) a.out_status[b] = cd.bad_n;
    }
}

// Zeroes request b's tile records in the workspace once the fold has read
// them (every thread of the workgroup, after the fold's barrier), leaving the
// workspace zero for the next call.
__device__ inline void clear_records(const Args& a, int b) {
    Seg* r = a.segs + (size_t)b * a.R * a.tpr;
    for (int i = threadIdx.x; i < a.R * a.tpr; i += blockDim.x) r[i] = Seg{0.f, 0, 0.0};
}

// -------------------------------------------------------------- decide
// The greedy rule's decide workgroup folds only K + 1 rows: eight waves take
// them in one batch for K < 8 and launch faster than sixteen.
constexpr int decide_threads(int mode) { return mode == kGreedy ? 512 : kDecideThreads; }

// Greedy: wave 0 takes the decision from the folded rows; the workgroup
// writes the accepted prefix, and position n gets the argmax of target row n
// (the correction after a mismatch, or the bonus token).
__device__ void greedy_finish(const Args& a, int b, const RowStats& rs, const ChainVals& cv) {
    __shared__ ChainDecision cd;
    if (threadIdx.x < 64) chain_decide<kGreedy>(a, rs, cv, cd);
    __syncthreads();
    write_prefix<kGreedy>(a, b, cd);
    if (threadIdx.x == 0) {
        const int n = cd.n;
        a.out_tok[(size_t)b * a.L + n] = rs.g[n];
        if (a.out_tlp) a.out_tlp[(size_t)b * a.L + n] = (float)(-rs.lnS[n]);
        if (a.out_blp) a.out_blp[(size_t)b * a.L + n] = 0.f;
    }
}

// Tree: wave 0 (lane i = node i) finds the deepest accepted node from the
// rows' argmax (rs.g) by pointer jumping and walks its path; the workgroup
// writes the outputs (NT threads).  p and t: node threadIdx.x's parent and
// token (threads 1 <= i < N), loaded before the fold; nraw the node count.
// Rows past the node count are never consulted (a parent index is below its
// child's).
template <int NT>
__device__ void tree_finish(const Args& a, int b, const RowStats& rs, int nraw, int p, int t) {
    __shared__ int t_par[SPEC_MAX_NODES];
    __shared__ int t_tok[SPEC_MAX_NODES];
    __shared__ int t_path[SPEC_MAX_NODES];
    __shared__ int t_d, t_e, t_bad;
    const int N = a.rows_t;
    const int nb = min(max(nraw, 1), N);
    if (threadIdx.x < 64) {
        // wave 0, lane i = node i.  Pointer jumping: `ok` says every node
        // from i up to (not including) `anc` matches, `dep` counts those
        // edges; each round doubles the span, so six rounds reach the root
        // from any depth below 64.  A node that does not match (or is
        // malformed, or lies beyond the tree) stops its chain with ok =
        // false, which its descendants inherit.
        const int i = threadIdx.x;
        bool bad = false, match = false;
        int par = -1;
        if (i >= 1 && i < nb) {
            bad = !(p >= 0 && p < i && (unsigned)t < (unsigned)a.Vtot);
            par = bad ? -1 : p;
            match = !bad && (t == rs.g[p]);
        }
        t_par[i] = par;
        t_tok[i] = t;
        const unsigned long long bm = __ballot(bad);
        bool ok = (i == 0) || match;
        int anc = match ? par : -1;
        int dep = (i == 0) ? 0 : 1;
#pragma unroll
        for (int round = 0; round < 6; ++round) {
            const int src = anc >= 0 ? anc : i;
            const int ok_a = __shfl(ok ? 1 : 0, src);
            const int dep_a = __shfl(dep, src);
            const int anc_a = __shfl(anc, src);
            if (anc >= 0) {
                ok = ok && ok_a;
                dep += dep_a;
                anc = anc_a;
            }
        }
        // deepest accepted node, ties to the lowest index (the root is
        // always accepted at depth 0)
        const int key = ok ? (dep << 6) | (63 - i) : -1;
        const int kmax = wave_max_i(key);
        const int e = 63 - (kmax & 63), d = kmax >> 6;
        int v = e;
        for (int k = d - 1; k >= 0; --k) {
            if (i == 0) t_path[k] = v;
            v = __builtin_amdgcn_readlane(par, v);
        }
        if (i == 0) {
            t_bad = bm != 0ull;
            t_d = d;
            t_e = e;
        }
    }
    __syncthreads();
    const int d = t_d, e = t_e;
    for (int k = threadIdx.x; k < N; k += NT) {
        int32_t* otok = a.out_tok + (size_t)b * N;
        if (k < d) {
            const int v = t_path[k];
            a.out_path[(size_t)b * N + k] = v;
            otok[k] = t_tok[v];
            if (a.out_tlp) a.out_tlp[(size_t)b * N + k] = (float)(-rs.lnS[t_par[v]]);
        } else {
            a.out_path[(size_t)b * N + k] = -1;
            otok[k] = (k == d) ? rs.g[e] : -1;
            if (a.out_tlp) a.out_tlp[(size_t)b * N + k] = (k == d) ? (float)(-rs.lnS[e]) : 0.f;
        }
        if (a.out_blp) a.out_blp[(size_t)b * N + k] = 0.f;
    }
    if (threadIdx.x == 0) {
        a.out_len[b] = d;
        a.out_status[b] = t_bad;
    }
}

// Greedy and tree: one workgroup (decide_threads) per request folds the tile
// records (one row per wave), takes the decision and writes the outputs.
template <typename T, int MODE, bool SUM, bool SHARD>
__global__ __launch_bounds__(decide_threads(MODE)) void k_decide(const Args a) {
    constexpr int NT = decide_threads(MODE);
    constexpr int NW = NT / 64;
    const int b = blockIdx.x;
    __shared__ double tab[kExpTab];
    __shared__ RowStats rs;
    if (SUM) fill_exp_table(tab);
    if constexpr (MODE == kGreedy) {
        ChainVals cv;
        if (threadIdx.x < 64) chain_load_tokens<MODE>(a, b, cv);
        fold_rows<MODE, SUM, NW, SHARD>(a, b, a.R, rs, tab, [&]() {
            if (threadIdx.x < 64) chain_load_values<T, MODE, SHARD>(a, b, cv);
            __syncthreads();  // the exp table; every load above is in flight
        });
        if (!SHARD) clear_records(a, b);
        greedy_finish(a, b, rs, cv);
        return;
    } else {
        // tree: a node is accepted iff its token is its parent's argmax and
        // its parent is accepted; parents precede children
        const int N = a.rows_t;
        // the node count, parents and tokens are loaded together, before the
        // fold, which takes every row of the request: records of rows past
        // the node count are stale but never consulted (a parent index is
        // below its child's)
        const int nraw = a.num_nodes ? a.num_nodes[b] : N;
        int p = -1, t = -1;
        if (threadIdx.x >= 1 && (int)threadIdx.x < N) {
            p = a.parents[b * N + threadIdx.x];
            t = a.tok[b * N + threadIdx.x];
        }
        fold_rows<kTree, SUM, NW, SHARD>(a, b, N, rs, tab, [] {
            __syncthreads();  // the exp table; every load above is in flight
        });
        if (!SHARD) clear_records(a, b);
        tree_finish<NT>(a, b, rs, nraw, p, t);
    }
}

// This thread's share of the fp64 sums of chunk c of the terminal row(s) of
// request b: exp(l - Mt) and exp(d - Md) over its tokens, and over those
// classified p > q against the threshold cls, with the smallest distance of
// (l - Mt) - (d - Md) from cls.  Thread tid of kThreads covers the tokens
// c*kChunk + (k*kThreads + tid)*VEC + [0, VEC) for k < kRun/VEC; a thread
// past the row's end reads nothing (its loads are masked).
struct ChunkPartial {
    double sa, sb, pa, pb, dmin;
};
template <typename T>
__device__ inline ChunkPartial chunk_partial(const Args& a, int b, int n, bool residual, double Mt,
                                             double Md, double cls, int c, int tid, const double* tab) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NV = kRun / VEC;  // 16-byte vectors per thread per chunk
    const T* trow = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + n) * a.V;
    const T* drow = residual ? reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + n) * a.V : trow;
    const __amdgpu_buffer_rsrc_t rt = row_rsrc(trow, a.V);
    const __amdgpu_buffer_rsrc_t rd = row_rsrc(drow, a.V);
    const int c0 = c * kChunk;
    const int c1 = min(c0 + kChunk, a.V);
    u32x4 qt[NV], qd[NV];
    ChunkPartial p = {0.0, 0.0, 0.0, 0.0, INFINITY};
    if (residual) {  // uniform: one loop per case, no per-token branch
        load_chunk<T, NV>(rt, c0, c1, a.vec_t, tid, qt);
        load_chunk<T, NV>(rd, c0, c1, a.vec_d, tid, qd);
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const double xa = (double)Elem<T>::get(qt[k], i) - Mt;
                const double xb = (double)Elem<T>::get(qd[k], i) - Md;
                const double ea = exp_nonpos(xa, tab);
                const double eb = exp_nonpos(xb, tab);
                p.sa += ea;
                p.sb += eb;
                const double dd = (xa - xb) - cls;
                const double pq = (dd > 0.0) ? 1.0 : 0.0;  // p > q
                p.pa = fma(ea, pq, p.pa);
                p.pb = fma(eb, pq, p.pb);
                p.dmin = fmin(p.dmin, fabs(dd));
            }
    } else {
        load_chunk<T, NV>(rt, c0, c1, a.vec_t, tid, qt);
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int i = 0; i < VEC; ++i) p.sa += exp_nonpos((double)Elem<T>::get(qt[k], i) - Mt, tab);
    }
    return p;
}

// -------------------------------------------------------------------- pass 2
// Sweep: one workgroup per (request, 4096-token chunk).  Every workgroup of
// the request folds the tile records and takes the decision itself (same
// data, same order, same result), so no kernel boundary sits between the
// decision and the sweep; chunk 0 also writes the accepted prefix and the
// decision record.  Each workgroup then sums its chunk of the row(s) the
// terminal token is drawn from, in fp64.
template <typename T, int MODE, bool SHARD>
__global__ __launch_bounds__(kSweepThreads, kPass2WavesPerSimd) void k_sweep(const Args a) {
    constexpr bool EXACT = (MODE == kExact);
    constexpr int NW = kSweepThreads / 64;

    // kSweepGroups consecutive chunks per workgroup, one 256-thread group each
    const int wpr = (a.C2 + kSweepGroups - 1) / kSweepGroups;
    const int b = blockIdx.x / wpr;
    const int grp = (int)threadIdx.x / kThreads;
    const int c = (blockIdx.x - b * wpr) * kSweepGroups + grp;
    const int tid = (int)threadIdx.x - grp * kThreads;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    __shared__ double tab[kExpTab];
    __shared__ RowStats rs;
    __shared__ ChainDecision cd;
    __shared__ double red[NW][5];
    fill_exp_table(tab);
    ChainVals cv;
    if (threadIdx.x < 64) chain_load_tokens<MODE>(a, b, cv);
    fold_rows<MODE, true, NW, SHARD>(a, b, a.R, rs, tab, [&]() {
        if (threadIdx.x < 64) chain_load_values<T, MODE, SHARD>(a, b, cv);
        __syncthreads();  // the exp table; every load above is in flight
    });
    if (threadIdx.x < 64) chain_decide<MODE>(a, rs, cv, cd);
    __syncthreads();
    const int n = cd.n;
    const bool residual = EXACT && n < a.K;
    const double Mt = rs.M[n], Md = residual ? (double)rs.M[a.rows_t + n] : 0.0;
    // p > q  <=>  (l - Mt) - (d - Md) > lnSt - lnSd, with the streamed
    // normalizers
    const double cls = residual ? rs.lnS[n] - rs.lnS[a.rows_t + n] : 0.0;
    if (c == 0) {
        write_prefix<MODE>(a, b, cd);
        if (threadIdx.x == 0) {
            Decision d;
            d.n = n;
            d.residual = residual;
            d.pad0 = d.pad1 = 0;
            d.Mt = Mt;
            d.Md = Md;
            d.cls = cls;
            d.rn = cd.r[n < a.K ? n : 0];
            a.dec[b] = d;
        }
    }
    const ChunkPartial cp = chunk_partial<T>(a, b, n, residual, Mt, Md, cls, c, tid, tab);
    double sa = cp.sa, sb = cp.sb, pa = cp.pa, pb = cp.pb, dmin = cp.dmin;
    sa = wave_sum(sa);
    if (residual) {
        sb = wave_sum(sb);
        pa = wave_sum(pa);
        pb = wave_sum(pb);
        dmin = wave_min_d(dmin);
    }
    if (lane == 0) {
        red[wave][0] = sa;
        red[wave][1] = sb;
        red[wave][2] = pa;
        red[wave][3] = pb;
        red[wave][4] = dmin;
    }
    __syncthreads();
    if (tid == 0 && c < a.C2) {
        ChunkSums cs = {0.0, 0.0, 0.0, 0.0, INFINITY, 0.0};
        for (int w = grp * kWaves; w < (grp + 1) * kWaves; ++w) {
            cs.sa += red[w][0];
            cs.sb += red[w][1];
            cs.pa += red[w][2];
            cs.pb += red[w][3];
            cs.dmin = fmin(cs.dmin, red[w][4]);
        }
        a.sums[(size_t)b * a.C2 + c] = cs;
    }
}

// Terminal sample: one workgroup per request (the kernel boundary makes the
// chunk sums visible).  Wave 0 turns the chunk sums into chunk masses of
// relu(p - q) (or of p), scans them and finds the chunk holding u_K * Z; the
// workgroup (1024 threads, four consecutive tokens each) then rescans that
// chunk with a block scan and writes the terminal token and its log-probs.
//
// Sharded: lane l of wave 0 holds chunk l % C2 of shard l / C2 (the gathered
// slots, in shard order, tile the vocabulary in ascending order); only the
// shard whose chunk holds the draw rescans it.
template <typename T, int MODE, bool SHARD>
__global__ __launch_bounds__(kSampleThreads) void k_sample(const Args a) {
    constexpr bool EXACT = (MODE == kExact);
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = threadIdx.x;

    __shared__ double tab[kExpTab];
    __shared__ int s_cstar, s_res;
    __shared__ double s_base, s_target, s_iS, s_iSq, s_lnS, s_lnZ, s_l1r;
    __shared__ double s_wtot[kSampleWaves];
    __shared__ int s_pick[kSampleWaves][3];
    fill_exp_table(tab);

    const Decision dc = a.dec[b];
    const int n = dc.n;
    const bool residual = EXACT && dc.residual;
    const double Md = dc.Md, cls = dc.cls;
    // Chunk masses of a residual draw whose classification must be redone
    // (see below), the exact threshold, and the chunks concerned.
    __shared__ double s_W[64];
    __shared__ double s_cls;
    __shared__ unsigned long long s_sus;
    double S0 = 1.0, Z0 = 1.0;  // wave 0: the normalizer and the terminal draw's total
    const int nchunk = SHARD ? a.G * a.C2 : a.C2;
    ChunkSums cs = {0.0, 0.0, 0.0, 0.0, INFINITY, 0.0};  // wave 0, lane l: chunk l
    double S = 1.0, iS = 1.0, iSq = 1.0;
    // Wave 0: the draw's total Z from the chunk masses W (lane = chunk), a wave
    // scan, and the chunk whose interval holds u_K * Z.
    auto pick = [&](double W) {
        const double Zr = residual ? wave_sum(W) : 0.0;
        const bool res = residual && (Zr > 0.0);
        if (residual && !res) W = cs.sa;  // relu(p - q) has no mass: draw from p
        const double Z = res ? Zr : S;
        const double target = (double)a.u[b * (a.K + 1) + a.K] * Z;
        const double incl = wave_incl_scan(W);
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;  // [excl, incl) of consecutive chunks tile [0, Z)
        const bool has = lane < nchunk && W > 0.0;
        const unsigned long long mine = __ballot(has && excl <= target && target < incl);
        const unsigned long long hasm = __ballot(has);
        // the unique chunk whose interval holds target; if rounding pushed
        // target past the last boundary, the last chunk with mass
        const int cstar = mine ? __builtin_ctzll(mine) : (hasm ? 63 - __builtin_clzll(hasm) : 0);
        const double base = readlane_d(excl, cstar);
        S0 = S;
        Z0 = Z;
        if (lane == 0) {
            s_cstar = cstar;
            s_base = base;
            s_target = target;
            s_res = res;
        }
    };
    if (wave == 0) {
        if (lane < nchunk) {
            const ChunkSums* src = a.sums + (size_t)b * a.C2 + lane;
            if (SHARD) {  // slot sl starts sl * sums_slot bytes in
                const int sl = lane / a.C2;
                src = reinterpret_cast<const ChunkSums*>(reinterpret_cast<const unsigned char*>(a.sums) +
                                                         (size_t)sl * a.sums_slot) +
                      (size_t)b * a.C2 + (lane - sl * a.C2);
            }
            cs = *src;
        }
        S = wave_sum(cs.sa);
        const double Sq = residual ? wave_sum(cs.sb) : 1.0;
        iS = 1.0 / S;
        iSq = 1.0 / Sq;
        // residual mass of the chunk (clamped: rounding can leave a
        // rounding-size negative)
        const double W = residual ? fmax(cs.pa * iS - cs.pb * iSq, 0.0) : cs.sa;
        // The sweep classified tokens p > q against the streamed normalizers;
        // the exact threshold comes from the fp64 sums just formed.  A token
        // the two thresholds classify differently lies between them, so only
        // chunks with a token that close (plus a rounding allowance) need
        // their mass recomputed.  Vocabulary shards keep the streamed
        // threshold (their columns are not all here).
        double clsx = cls;
        unsigned long long sus = 0ull;
        if (EXACT && !SHARD && residual) {
            clsx = log(S) - log(Sq);
            const double gap = fabs(clsx - cls) + 1e-12;
            sus = __ballot(lane < nchunk && cs.dmin <= gap);
        }
        if (lane == 0) {
            s_cls = clsx;
            s_sus = sus;
            s_iS = iS;
            s_iSq = iSq;
        }
        if (sus) {
            s_W[lane] = W;
        } else {
            pick(W);
        }
    }
    __syncthreads();
    if (s_sus) {  // workgroup-uniform and rare: recompute those chunks' masses
        const T* tr = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + n) * a.V;
        const T* dr = reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + n) * a.V;
        const double clsx = s_cls, jS = s_iS, jSq = s_iSq;
        for (unsigned long long m = s_sus; m; m &= m - 1) {
            const int c = __builtin_ctzll(m);
            const int e = c * kChunk + t * kSampleRun;
            float lt[kSampleRun], ld[kSampleRun];
            Elem<T>::load4(row_rsrc(tr, a.V), e, a.V, a.vec_t, lt);
            Elem<T>::load4(row_rsrc(dr, a.V), e, a.V, a.vec_d, ld);
            double sum = 0.0;
#pragma unroll
            for (int i = 0; i < kSampleRun; ++i) {
                const double xa = (double)lt[i] - dc.Mt, xb = (double)ld[i] - Md;
                if (xa - xb > clsx) sum += fmax(exp_nonpos(xa, tab) * jS - exp_nonpos(xb, tab) * jSq, 0.0);
            }
            sum = wave_sum(sum);
            if (lane == 0) s_wtot[wave] = sum;
            __syncthreads();
            if (t == 0) {
                double z = 0.0;
                for (int ww = 0; ww < kSampleWaves; ++ww) z += s_wtot[ww];
                s_W[c] = z;
            }
            __syncthreads();
        }
        if (wave == 0) pick(s_W[lane]);
        __syncthreads();
    }

    const double Mt = dc.Mt;
    int cstar = s_cstar;
    if (SHARD) {
        const int owner = cstar / a.C2;
        if (threadIdx.x == 0 && a.out_owner) a.out_owner[b] = owner;
        if (owner != a.shard) return;  // uniform: another shard draws
        cstar -= owner * a.C2;
    }
    const bool res = s_res;
    const double target = s_target, clsx = s_cls;
    iS = s_iS;
    iSq = s_iSq;
    const T* trow = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + n) * a.V;
    const T* drow = residual ? reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + n) * a.V : trow;
    const int e0 = cstar * kChunk + t * kSampleRun;
    float lt[kSampleRun], ld[kSampleRun];
    Elem<T>::load4(row_rsrc(trow, a.V), e0, a.V, a.vec_t, lt);
    Elem<T>::load4(row_rsrc(drow, a.V), e0, a.V, residual ? a.vec_d : a.vec_t, ld);
    // the logs of the outputs, while the chunk loads are in flight (the last
    // barrier below publishes them)
    if (t == 0) {
        s_lnS = log(S0);
        s_lnZ = log(Z0);
        s_l1r = res ? log1p(-dc.rn) : 0.0;
    }
    double w[kSampleRun];
    double tsum = 0.0;
    unsigned pos = 0u, fin = 0u;  // bit i: token i has mass / a finite logit
#pragma unroll
    for (int i = 0; i < kSampleRun; ++i) {
        const double xa = (double)lt[i] - Mt;
        const double ea = exp_nonpos(xa, tab);
        double wi = ea;
        if (res) {
            const double xb = (double)ld[i] - Md;
            const double eb = exp_nonpos(xb, tab);
            wi = (xa - xb > clsx) ? fmax(ea * iS - eb * iSq, 0.0) : 0.0;
        }
        w[i] = wi;
        tsum += wi;
        pos |= (wi > 0.0) ? (1u << i) : 0u;
        fin |= (lt[i] > -INFINITY) ? (1u << i) : 0u;
    }
    // block scan in thread order; the exclusive prefix of a thread is the
    // previous thread's inclusive prefix, bit for bit
    const double wincl = wave_incl_scan(tsum);
    if (lane == 63) s_wtot[wave] = wincl;
    __syncthreads();
    // offset of this wave: the earlier waves' totals added in wave order (all
    // read at once, then summed)
    double tot[kSampleWaves];
#pragma unroll
    for (int ww = 0; ww < kSampleWaves; ++ww) tot[ww] = s_wtot[ww];
    double off = 0.0;
#pragma unroll
    for (int ww = 0; ww < kSampleWaves; ++ww)
        if (ww < wave) off += tot[ww];
    const double tincl = wincl + off;
    double texcl = __shfl_up(tincl, 1);
    if (lane == 0) texcl = off;
    // first crossing of the running sum past target in this thread's tokens
    double cum = s_base + texcl;
    int cand = INT_MAX;
#pragma unroll
    for (int i = 0; i < kSampleRun; ++i) {
        if (w[i] > 0.0 && cand == INT_MAX) {
            cum += w[i];
            if (cum > target) cand = e0 + i;
        }
    }
    const int lastpos = pos ? e0 + 31 - __builtin_clz(pos) : -1;
    const int anypos = fin ? e0 + 31 - __builtin_clz(fin) : -1;
    const int wc = wave_min_i(cand), wl = wave_max_i(lastpos), wa = wave_max_i(anypos);
    if (lane == 0) {
        s_pick[wave][0] = wc;
        s_pick[wave][1] = wl;
        s_pick[wave][2] = wa;
    }
    __syncthreads();
    int yc = INT_MAX, yl = -1, ya = -1;
#pragma unroll
    for (int ww = 0; ww < kSampleWaves; ++ww) {
        yc = min(yc, s_pick[ww][0]);
        yl = max(yl, s_pick[ww][1]);
        ya = max(ya, s_pick[ww][2]);
    }
    // The crossing token; if rounding left none, the last token with mass in
    // the chunk; if the chunk had none, its last finite token.  Always a valid
    // index.
    int y = (yc != INT_MAX) ? yc : (yl >= 0 ? yl : ya);
    if (y < 0 || y >= a.V) y = 0;
    const int rel = y - cstar * kChunk;
    const bool inchunk = rel >= 0 && rel < kChunk;
    if (t == (inchunk ? rel / kSampleRun : 0)) {
        float ly = lt[0];
        double wy = w[0];
        if (inchunk) {
#pragma unroll
            for (int i = 1; i < kSampleRun; ++i)
                if (e0 + i == y) {
                    ly = lt[i];
                    wy = w[i];
                }
        } else {
            ly = Elem<T>::at(trow, (size_t)y);
            const float dy = Elem<T>::at(drow, (size_t)y);
            const double xa = (double)ly - Mt, xb = (double)dy - Md;
            wy = 0.0;
            if (res && xa - xb > clsx) wy = fmax(exp_nonpos(xa, tab) * iS - exp_nonpos(xb, tab) * iSq, 0.0);
        }
        const int L = a.L;
        a.out_tok[(size_t)b * L + n] = SHARD ? y + a.shard * a.V : y;
        const double tlp = ((double)ly - Mt) - s_lnS;
        // behaviour log-prob: residual draw, power-rule fallback after a
        // rejection (1 - a_n) p_n(y), or a plain draw from p
        const double blp = res ? s_l1r + log(wy) - s_lnZ
                               : ((MODE == kPower && n < a.K) ? log1p(-dc.rn) + tlp : tlp);
        if (a.out_tlp) a.out_tlp[(size_t)b * L + n] = (float)tlp;
        if (a.out_blp) a.out_blp[(size_t)b * L + n] = (float)blp;
    }
}

// ------------------------------------------------------------ single launch
// The exact, relaxed and power rules run as one launch per call, with no
// kernel boundary between the stream and the terminal draw.  The launch's
// first nstream workgroups stream tiles (stream_tile, records published).
// Behind them, one sweep workgroup per (request, 2048- or 4096-token chunk)
// waits for its request's row records (folded once per row by the request's
// first sweep workgroups) and takes the decision (the same decision in every
// workgroup of the request), writes the accepted prefix (chunk 0), sums its
// chunk of the terminal row(s) in fp64 and publishes the sums.  The
// request's last sweep workgroup then waits for all of the request's chunk
// sums, draws the terminal token
// (draw_terminal) and zeroes the request's published words for the next
// call: every other workgroup of the request has read the records before it
// published its sums.

// A sweep record holds the chunk's exp sums of the target and draft rows (S,
// Sq), dmin (see ChunkSums), then per 1024-token sub-chunk the two sums the
// draw's mass is formed from (target and draft exp sums over the tokens
// classified p > q for a residual draw, the target exp sum otherwise).

// Drafted-token logits read from the inputs (the token is loaded first, so
// these loads wait for it; they overlap the wait for the records).
template <typename T, int MODE>
__device__ inline void chain_load_inputs(const Args& a, int b, ChainVals& cv) {
    const int j = threadIdx.x;
    if (j < a.K) {
        cv.bad = (unsigned)cv.x >= (unsigned)a.V;
        if (MODE == kGreedy || cv.bad) return;
        cv.lx = Elem<T>::at(reinterpret_cast<const T*>(a.T), (size_t)(b * a.rows_t + j) * a.V + cv.x);
        if (uses_draft(MODE))
            cv.dx = Elem<T>::at(reinterpret_cast<const T*>(a.D), (size_t)(b * a.K + j) * a.V + cv.x);
    }
}

// Weight of one token in the terminal draw: exp(l - Mt) from p, or for the
// residual relu(p - q) = max(p - q, 0) with p > q decided by the threshold
// clsx on (l - Mt) - (d - Md).  One expression wherever a weight is formed.
__device__ inline double draw_weight(bool res, float l, float d, double Mt, double Md, double clsx,
                                     double iS, double iSq, const double* tab) {
    const double xa = (double)l - Mt;
    const double ea = exp_nonpos(xa, tab);
    if (!res) return ea;
    const double xb = (double)d - Md;
    if (!(xa - xb > clsx)) return 0.0;
    return fmax(fma(ea, iS, -(exp_nonpos(xb, tab) * iSq)), 0.0);
}

// Zeroes request b's published row and chunk records (every thread; after
// all of the request's reads of them).  Its tile records were zeroed by the
// workgroups that folded them.
__device__ inline void clear_published(const Args& a, int b, int sums_words) {
    uint64_t* r = a.frow + (size_t)b * a.R * 2;
    for (int i = threadIdx.x; i < a.R * 2; i += blockDim.x) store_word(r + i, 0ull);
    uint64_t* m = a.fsums + (size_t)b * sums_words;
    for (int i = threadIdx.x; i < sums_words; i += blockDim.x) store_word(m + i, 0ull);
}

// The terminal draw of request b, by its last sweep workgroup.  Wave 0 waits
// for the request's published sweep records (lane l = draw chunk l of 4096
// tokens: one record, or two of 2048 tokens), forms S,
// Sq, the exact p > q threshold and the sub-chunk masses, recomputes the
// masses of chunks the streamed threshold may have classified otherwise,
// scans the chunks and then the sub-chunks of the chunk holding u_K * Z.
// The workgroup rescans that sub-chunk, four consecutive tokens per thread,
// with a block scan, and writes the terminal token and its log-probs.
template <typename T, int MODE, int PER>
__device__ void draw_terminal(const Args& a, const int b, const ChainDecision& cd, const RowStats& rs,
                              const double* tab) {
    constexpr bool EXACT = (MODE == kExact);
    constexpr int NT = kThreads, NWV = NT / 64, RUN = kSub / NT;
    static_assert(RUN == 4, "four tokens per thread (one load4 per row)");
    constexpr int RPL = kSweepSplit / PER;     // sweep records per draw chunk (lane)
    constexpr int WPR = sweep_words(PER);      // words per record
    constexpr int SPR = PER * kSweepSubs;      // sub-chunks per record
    const int nrec = (a.C2s + PER - 1) / PER;  // the request's sweep records
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
    const int n = cd.n;
    const bool residual = EXACT && n < a.K;
    const double Mt = rs.M[n];
    const double Md = residual ? (double)rs.M[a.rows_t + n] : 0.0;
    const double cls = residual ? rs.lnS[n] - rs.lnS[a.rows_t + n] : 0.0;
    const double rn = cd.r[n < a.K ? n : 0];
    const T* trow = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + n) * a.V;
    const T* drow = residual ? reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + n) * a.V : trow;
    const __amdgpu_buffer_rsrc_t rt = row_rsrc(trow, a.V);
    const __amdgpu_buffer_rsrc_t rd = row_rsrc(drow, a.V);

    __shared__ int s_sub, s_res, s_ok;
    __shared__ double s_base, s_target, s_iS, s_iSq, s_lnS, s_lnZ, s_l1r, s_cls;
    __shared__ double s_wtot[NWV];
    __shared__ int s_pick[NWV][3];
    __shared__ double s_W[64][kSubs];
    __shared__ unsigned long long s_sus;

    // wave 0, lane l: chunk l's target exp sum (the fallback's p mass per
    // sub-chunk is kept in s_W when needed) and the draw's normalizers
    double S0 = 1.0, Z0 = 1.0;
    double S = 1.0;
    double pm[kSubs];  // wave 0, lane l: chunk l's p mass per sub-chunk (non-residual) or unused
    // Wave 0: the draw's total from the sub-chunk masses W[] (lane = chunk),
    // a scan over chunks, then over the sub-chunks of the chunk holding
    // u_K * Z.
    auto pick = [&](const double (&W)[kSubs], const double (&P)[kSubs]) {
        double wc = 0.0;
#pragma unroll
        for (int k = 0; k < kSubs; ++k) wc += W[k];
        const double Zr = residual ? wave_sum(wc) : 0.0;
        const bool res = residual && (Zr > 0.0);
        double Wk[kSubs];
#pragma unroll
        for (int k = 0; k < kSubs; ++k) Wk[k] = (residual && !res) ? P[k] : W[k];  // no residual mass: draw from p
        double cw = 0.0;
#pragma unroll
        for (int k = 0; k < kSubs; ++k) cw += Wk[k];
        const double Z = res ? Zr : S;
        const double target = (double)a.u[b * (a.K + 1) + a.K] * Z;
        const double incl = wave_incl_scan(cw);
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;  // [excl, incl) of consecutive chunks tile [0, Z)
        const bool has = lane < a.C2 && cw > 0.0;
        const unsigned long long mine = __ballot(has && excl <= target && target < incl);
        const unsigned long long hasm = __ballot(has);
        // the unique chunk whose interval holds target; if rounding pushed
        // target past the last boundary, the last chunk with mass
        const int cstar = mine ? __builtin_ctzll(mine) : (hasm ? 63 - __builtin_clzll(hasm) : 0);
        // within it, the sub-chunk whose interval holds target, or its last
        // sub-chunk with mass (lane cstar decides, in sub-chunk order)
        int sub = 0;
        double base = excl;
        if (lane == cstar) {
            double run = excl;
            int last = -1, hit = -1;
            double hbase = excl, lbase = excl;
#pragma unroll
            for (int k = 0; k < kSubs; ++k) {
                if (Wk[k] > 0.0) {
                    if (hit < 0 && target < run + Wk[k]) {
                        hit = k;
                        hbase = run;
                    }
                    last = k;
                    lbase = run;
                }
                run += Wk[k];
            }
            sub = hit >= 0 ? hit : (last >= 0 ? last : 0);
            base = hit >= 0 ? hbase : lbase;
        }
        sub = __builtin_amdgcn_readlane(sub, cstar);
        base = readlane_d(base, cstar);
        S0 = S;
        Z0 = Z;
        if (lane == 0) {
            s_sub = cstar * kSubs + sub;
            s_base = base;
            s_target = target;
            s_res = res;
        }
    };
    if (wave == 0) {
        bool ok = true;
        // lane l: the records RPL*l + j of draw chunk l that exist
        uint64_t w[RPL][WPR];
        bool have[RPL];
        const uint64_t* src[RPL];
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int cs = RPL * lane + j;
            have[j] = lane < a.C2 && cs < nrec;
            src[j] = a.fsums + ((size_t)b * nrec + (have[j] ? cs : 0)) * WPR;
#pragma unroll
            for (int i = 0; i < WPR; ++i) w[j][i] = kTop;  // absent: zero sums
        }
        // the other chunks' workgroups may still be summing: first wait for
        // every record's first word (one load per record a round), then read
        // all words (every word each round, the round's loads in flight
        // together) until none is missing
        for (int it = 0, all = 0;; ++it) {
            bool missing = false;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                if (!have[j]) continue;
                if (all) {
#pragma unroll
                    for (int i = 0; i < WPR; ++i) w[j][i] = load_word(src[j] + i);
                } else {
                    w[j][0] = load_word(src[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                if (!have[j]) continue;
                if (all) {
#pragma unroll
                    for (int i = 0; i < WPR; ++i) missing |= w[j][i] == 0ull;
                } else {
                    missing |= w[j][0] == 0ull;
                }
            }
            const bool none = __ballot(missing) == 0ull;
            if (none && all) break;
            if (none) {
                all = 1;
                continue;
            }
            if (it >= a.spin_limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        const bool all_ok = __ballot(!ok) == 0ull;
        double sa = 0.0, sb = 0.0, dmin = INFINITY;
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            sa += dec_nonneg(w[j][0]);
            sb += dec_nonneg(w[j][1]);
            if (have[j]) dmin = fmin(dmin, dec_nonneg(w[j][2]));
        }
        S = wave_sum(sa);
        const double Sq = residual ? wave_sum(sb) : 1.0;
        const double iS = 1.0 / S, iSq = 1.0 / Sq;
        double W[kSubs];
#pragma unroll
        for (int k = 0; k < kSubs; ++k) {
            const int j = k / SPR, kk = k - j * SPR;
            const double A = dec_nonneg(w[j][3 + 2 * kk]), Bq = dec_nonneg(w[j][4 + 2 * kk]);
            // residual mass of the sub-chunk (clamped: rounding can leave a
            // rounding-size negative), or its p mass
            W[k] = residual ? fmax(A * iS - Bq * iSq, 0.0) : A;
            pm[k] = residual ? 0.0 : A;
        }
        // The sweep classified tokens p > q against the streamed normalizers;
        // the exact threshold comes from the fp64 sums.  A token the two
        // thresholds classify differently lies between them, so only chunks
        // holding a token that close (plus a rounding allowance) need their
        // masses recomputed.
        double clsx = cls;
        unsigned long long sus = 0ull;
        if (residual) {
            clsx = log(S) - log(Sq);
            const double gap = fabs(clsx - cls) + 1e-12;
            sus = __ballot(lane < a.C2 && dmin <= gap);
        }
        if (lane == 0) {
            s_ok = all_ok;
            s_cls = clsx;
            s_sus = all_ok ? sus : 0ull;
            s_iS = iS;
            s_iSq = iSq;
        }
        if (all_ok) {
            if (sus || residual) {
                // the residual's fallback (no mass) draws from p: keep the
                // p masses too
#pragma unroll
                for (int k = 0; k < kSubs; ++k) s_W[lane][k] = W[k];
            }
            if (!sus) pick(W, pm);
        }
    }
    __syncthreads();
    if (!s_ok) {  // a chunk's sums never arrived: report, leave the words as they are
        if (t == 0) a.out_status[b] = 2;
        return;
    }
    const double clsx = s_cls, iS = s_iS, iSq = s_iSq;
    if (s_sus) {  // workgroup-uniform and rare: recompute those chunks' sub-chunk masses
        for (unsigned long long m = s_sus; m; m &= m - 1) {
            const int c = __builtin_ctzll(m);
            for (int k = 0; k < kSubs; ++k) {
                const int e = c * kChunk + k * kSub + t * RUN;
                float lt[RUN], ld[RUN];
                Elem<T>::load4(rt, e, a.V, a.vec_t, lt);
                Elem<T>::load4(rd, e, a.V, a.vec_d, ld);
                double sum = 0.0;
#pragma unroll
                for (int i = 0; i < RUN; ++i) sum += draw_weight(true, lt[i], ld[i], Mt, Md, clsx, iS, iSq, tab);
                sum = wave_sum(sum);
                if (lane == 0) s_wtot[wave] = sum;
                __syncthreads();
                if (t == 0) {
                    double z = 0.0;
                    for (int ww = 0; ww < NWV; ++ww) z += s_wtot[ww];
                    s_W[c][k] = z;
                }
                __syncthreads();
            }
        }
        if (wave == 0) {
            double W[kSubs];
#pragma unroll
            for (int k = 0; k < kSubs; ++k) W[k] = s_W[lane][k];
            pick(W, pm);
        }
        __syncthreads();
    }

    const int sub = s_sub;
    const bool res = s_res;
    const double target = s_target;
    const int e0 = sub * kSub + t * RUN;
    float lt[RUN], ld[RUN];
    Elem<T>::load4(rt, e0, a.V, a.vec_t, lt);
    Elem<T>::load4(rd, e0, a.V, residual ? a.vec_d : a.vec_t, ld);
    // the logs of the outputs, while the loads are in flight (the next
    // barrier publishes them)
    if (t == 0) {
        s_lnS = log(S0);
        s_lnZ = log(Z0);
        s_l1r = res ? log1p(-rn) : 0.0;
    }
    double w[RUN];
    double tsum = 0.0;
    unsigned pos = 0u, fin = 0u;  // bit i: token i has mass / a finite logit
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        w[i] = draw_weight(res, lt[i], ld[i], Mt, Md, clsx, iS, iSq, tab);
        tsum += w[i];
        pos |= (w[i] > 0.0) ? (1u << i) : 0u;
        fin |= (lt[i] > -INFINITY) ? (1u << i) : 0u;
    }
    // block scan in thread order; the exclusive prefix of a thread is the
    // previous thread's inclusive prefix, bit for bit
    const double wincl = wave_incl_scan(tsum);
    if (lane == 63) s_wtot[wave] = wincl;
    __syncthreads();
    double off = 0.0;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww)
        if (ww < wave) off += s_wtot[ww];
    const double tincl = wincl + off;
    double texcl = __shfl_up(tincl, 1);
    if (lane == 0) texcl = off;
    // first crossing of the running sum past target in this thread's tokens
    double cum = s_base + texcl;
    int cand = INT_MAX;
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        if (w[i] > 0.0 && cand == INT_MAX) {
            cum += w[i];
            if (cum > target) cand = e0 + i;
        }
    }
    const int lastpos = pos ? e0 + 31 - __builtin_clz(pos) : -1;
    const int anypos = fin ? e0 + 31 - __builtin_clz(fin) : -1;
    const int wc = wave_min_i(cand), wl = wave_max_i(lastpos), wa = wave_max_i(anypos);
    if (lane == 0) {
        s_pick[wave][0] = wc;
        s_pick[wave][1] = wl;
        s_pick[wave][2] = wa;
    }
    __syncthreads();
    int yc = INT_MAX, yl = -1, ya = -1;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
        yc = min(yc, s_pick[ww][0]);
        yl = max(yl, s_pick[ww][1]);
        ya = max(ya, s_pick[ww][2]);
    }
    // The crossing token; if rounding left none, the last token with mass in
    // the sub-chunk; if it had none, its last finite token.  Always a valid
    // index.
    int y = (yc != INT_MAX) ? yc : (yl >= 0 ? yl : ya);
    if (y < 0 || y >= a.V) y = 0;
    const int rel = y - sub * kSub;
    const bool insub = rel >= 0 && rel < kSub;
    if (t == (insub ? rel / RUN : 0)) {
        float ly = lt[0], dy = ld[0];
        double wy = w[0];
        if (insub) {
#pragma unroll
            for (int i = 1; i < RUN; ++i)
                if (e0 + i == y) {
                    ly = lt[i];
                    dy = ld[i];
                    wy = w[i];
                }
        } else {
            ly = Elem<T>::at(trow, (size_t)y);
            dy = res ? Elem<T>::at(drow, (size_t)y) : 0.f;
            wy = draw_weight(res, ly, dy, Mt, Md, clsx, iS, iSq, tab);
        }
        (void)dy;
        const int L = a.L;
        a.out_tok[(size_t)b * L + n] = y;
        const double tlp = ((double)ly - Mt) - s_lnS;
        // behaviour log-prob: residual draw, power-rule fallback after a
        // rejection (1 - a_n) p_n(y), or a plain draw from p
        const double blp = res ? s_l1r + log(wy) - s_lnZ
                               : ((MODE == kPower && n < a.K) ? log1p(-rn) + tlp : tlp);
        if (a.out_tlp) a.out_tlp[(size_t)b * L + n] = (float)tlp;
        if (a.out_blp) a.out_blp[(size_t)b * L + n] = (float)blp;
        a.out_status[b] = cd.bad_n;
    }
    __syncthreads();  // every read of the request's published words is done
    clear_published(a, b, nrec * WPR);
}

// Row r of request b, by one wave: waits for the row's published tile
// records (lane = tile), folds them as fold_batches does (max with the
// lowest index of the max for the greedy rules or the rank count for the
// relaxed rule, and with SUM the fp64 sum rescaled to the row max),
// publishes the row's record {M, argmax or count, S} and zeroes the tile
// records.  Returns false (in every lane) if the wait ran out.
template <int MODE, bool SUM = true>
__device__ bool fold_publish_row(const Args& a, int b, int r, const double* tab) {
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    constexpr bool COUNT = (MODE == kRelaxed);
    const int lane = threadIdx.x & 63;
    const bool have = lane < a.tpr;
    uint64_t* src = a.frec + 2 * (((size_t)b * a.R + r) * a.tpr + (have ? lane : 0));
    uint64_t w0 = 0ull, w1 = 0ull;
    for (int it = 0;; ++it) {
        if (have) {  // both words each round, in flight together
            w0 = load_word(src);
            w1 = load_word(src + 1);
        }
        if (__ballot(have && (w0 == 0ull || w1 == 0ull)) == 0ull) break;
        if (it >= a.spin_limit) return false;
        __builtin_amdgcn_s_sleep(4);
    }
    const Seg sg = have ? decode_record(w0, w1) : neutral_record(ARGMAX);
    float M = sg.m;
    int ic = sg.ic;
    if (ARGMAX)
        wave_argmax(M, ic);
    else
        M = wave_max(M);
    if (COUNT) ic = wave_sum_i(ic);
    if (!ARGMAX && !COUNT) ic = 0;
    double S = 0.0;
    if (SUM) {
        // tile sum * 2^(fl(m*L) - M*L), exact reference difference in fp64
        double t = 0.0;
        if (sg.m > -INFINITY) {
            const float mL = sg.m * kLog2e;
            t = sg.s * exp_nonpos(((double)mL - (double)M * (double)kLog2e) * kLn2, tab);
        }
        S = wave_sum(t);
    }
    if (have) {  // read: zero them for the next call
        store_word(src, 0ull);
        store_word(src + 1, 0ull);
    }
    if (lane == 0) {
        Seg row;
        row.m = M;
        row.ic = ic;
        row.s = S;
        publish_record(a.frow + 2 * ((size_t)b * a.R + r), row);
    }
    return true;
}

// Row records 0..nrows-1 of request b into rs (lane = row, in waves 0 and
// 1; nrows <= 2 * 64): one lane waits for the last row's record, then the
// lanes read all of them, waiting for any still missing.  With SUM, lnS =
// log S per row, in parallel.  Returns false in a thread whose wait ran out.
// Ends with a barrier.
template <int MODE, bool SUM = true>
__device__ bool read_row_records(const Args& a, int b, RowStats& rs, int nrows) {
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    constexpr bool COUNT = (MODE == kRelaxed);
    const int tid = threadIdx.x;
    __shared__ int s_hint;
    bool ok = true;
    if (tid == 0) {
        s_hint = 1;
        const uint64_t* hint = a.frow + 2 * ((size_t)b * a.R + nrows - 1);
        for (int it = 0; load_word(hint) == 0ull; ++it) {
            if (it >= a.spin_limit) {
                s_hint = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
    }
    __syncthreads();
    if (!s_hint) ok = false;
    if (ok && tid < 128) {
        const bool have = tid < nrows;
        const uint64_t* src = a.frow + 2 * ((size_t)b * a.R + (have ? tid : 0));
        uint64_t w0 = 0ull, w1 = 0ull;
        for (int it = 0;; ++it) {
            if (have) {
                w0 = load_word(src);
                w1 = load_word(src + 1);
            }
            if (__ballot(have && (w0 == 0ull || w1 == 0ull)) == 0ull) break;
            if (it >= a.spin_limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (ok && have) {
            const Seg sg = decode_record(w0, w1);
            rs.M[tid] = sg.m;
            rs.g[tid] = ARGMAX ? sg.ic : 0;
            rs.c[tid] = COUNT ? sg.ic : 0;
            rs.lnS[tid] = SUM ? log(sg.s) : 0.0;
        }
    }
    __syncthreads();
    return ok;
}

// One sweep workgroup: request b, tokens [PER * kSweepChunk * c,
// PER * kSweepChunk * (c + 1)); publishes one record.  The first F =
// min(R, C2w) workgroups of every request fold its rows: they come first in
// index order, request by request (idx < B * F), so they start while the
// stream runs and fold each row as its tiles arrive; the request's other
// workgroups follow, request by request, and find the row records there.
template <typename T, int MODE, int PER>
__device__ void sweep_role(const Args& a, const int idx) {
    constexpr bool EXACT = (MODE == kExact);
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NV = PER * kSweepChunk / kThreads / VEC;  // 16-byte vectors per thread
    static_assert(NV * VEC * kThreads == PER * kSweepChunk && PER <= kSweepSplit, "whole vectors per thread");
    const int C2w = (a.C2s + PER - 1) / PER;  // sweep workgroups per request
    const int F = min(a.R, C2w);              // folding workgroups per request
    int b, c;
    if (idx < a.B * F) {
        b = idx / F;
        c = idx - b * F;
    } else {
        const int j = idx - a.B * F, nf = C2w - F;
        b = j / nf;
        c = F + (j - b * nf);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
    __shared__ double tab[kExpTab];
    __shared__ RowStats rs;
    __shared__ ChainDecision cd;
    __shared__ double red[kWaves][3 + 2 * NV];
    __shared__ int s_ok;
    // Each row of the request is folded once: the request's sweep workgroup
    // c takes rows c, c + C2w, ... (only the first R workgroups have one) and
    // publishes the row's record; then every sweep workgroup of the request
    // reads the R row records.  A workgroup waits only on streaming
    // workgroups, on its request's folding workgroups (which publish their
    // rows before they wait for anything but tiles, and start before every
    // non-folding workgroup), and the drawer on the request's other sweep
    // workgroups, which start before it.  The drafted tokens are loaded while the
    // exp table is computed, their logits (addresses depending on them)
    // while the row records are awaited.
    ChainVals cv;
    if (tid < 64) chain_load_tokens<MODE>(a, b, cv);
    if (tid == 0) s_ok = 1;
    fill_exp_table(tab);
    __syncthreads();  // the exp table, s_ok
    // (wave w takes the workgroup's rows w, w + kWaves, ...: with fewer
    // chunks than rows, a workgroup's rows are folded in parallel)
    for (int r = c + C2w * wave; r < a.R; r += C2w * kWaves)
        if (!fold_publish_row<MODE>(a, b, r, tab) && lane == 0) s_ok = 0;
    if (tid < 64) chain_load_inputs<T, MODE>(a, b, cv);
    if (!read_row_records<MODE>(a, b, rs, a.R)) s_ok = 0;
    __syncthreads();
    if (!s_ok) {  // a record never arrived: report, leave the words as they are
        if (tid == 0) a.out_status[b] = 2;
        return;
    }
    if (tid < 64) chain_decide<MODE>(a, rs, cv, cd);
    __syncthreads();
    const int n = cd.n;
    const bool residual = EXACT && n < a.K;
    const double Mt = rs.M[n], Md = residual ? (double)rs.M[a.rows_t + n] : 0.0;
    // p > q  <=>  (l - Mt) - (d - Md) > lnSt - lnSd, with the streamed normalizers
    const double cls = residual ? rs.lnS[n] - rs.lnS[a.rows_t + n] : 0.0;
    // the request's status is the drawing workgroup's: it succeeds only if
    // every sweep workgroup of the request did (it waits for all their sums)
    if (c == 0) write_prefix<MODE>(a, b, cd, false);

    // this thread's vectors k cover tokens c0 + (k*kThreads + tid)*VEC +
    // [0, VEC): vector k lies in sub-chunk ((k*kThreads + tid)*VEC) / kSub of
    // the workgroup's record
    const T* trow = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + n) * a.V;
    const T* drow = residual ? reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + n) * a.V : trow;
    const int c0 = c * PER * kSweepChunk, c1 = min(c0 + PER * kSweepChunk, a.V);
    u32x4 qt[NV], qd[NV];
    double sa = 0.0, sb = 0.0, dmin = INFINITY;
    double A[NV], Bq[NV];  // per vector: the sums its sub-chunk's mass is formed from
    if (residual) {
        load_chunk<T, NV>(row_rsrc(trow, a.V), c0, c1, a.vec_t, tid, qt);
        load_chunk<T, NV>(row_rsrc(drow, a.V), c0, c1, a.vec_d, tid, qd);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            A[k] = Bq[k] = 0.0;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const double xa = (double)Elem<T>::get(qt[k], i) - Mt;
                const double xb = (double)Elem<T>::get(qd[k], i) - Md;
                const double ea = exp_nonpos(xa, tab);
                const double eb = exp_nonpos(xb, tab);
                sa += ea;
                sb += eb;
                const double dd = (xa - xb) - cls;
                const double pq = (dd > 0.0) ? 1.0 : 0.0;  // p > q
                A[k] = fma(ea, pq, A[k]);
                Bq[k] = fma(eb, pq, Bq[k]);
                dmin = fmin(dmin, fabs(dd));
            }
        }
    } else {
        load_chunk<T, NV>(row_rsrc(trow, a.V), c0, c1, a.vec_t, tid, qt);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            A[k] = Bq[k] = 0.0;
#pragma unroll
            for (int i = 0; i < VEC; ++i) A[k] += exp_nonpos((double)Elem<T>::get(qt[k], i) - Mt, tab);
            sa += A[k];
        }
    }
    sa = wave_sum(sa);
    if (residual) {
        sb = wave_sum(sb);
        dmin = wave_min_d(dmin);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        A[k] = wave_sum(A[k]);
        if (residual) Bq[k] = wave_sum(Bq[k]);
    }
    if (lane == 0) {
        red[wave][0] = sa;
        red[wave][1] = sb;
        red[wave][2] = dmin;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            red[wave][3 + 2 * k] = A[k];
            red[wave][4 + 2 * k] = Bq[k];
        }
    }
    __syncthreads();
    if (tid == 0) {
        constexpr int WPR = sweep_words(PER);
        double v[WPR];
        v[0] = v[1] = 0.0;
        v[2] = INFINITY;
        for (int i = 3; i < WPR; ++i) v[i] = 0.0;
        for (int w = 0; w < kWaves; ++w) {
            v[0] += red[w][0];
            v[1] += red[w][1];
            v[2] = fmin(v[2], red[w][2]);
        }
        // sub-chunk sums in a fixed order: vector k, then wave
        for (int k = 0; k < NV; ++k)
            for (int w = 0; w < kWaves; ++w) {
                const int sc = ((k * kThreads + w * 64) * VEC) / kSub;
                v[3 + 2 * sc] += red[w][3 + 2 * k];
                v[4 + 2 * sc] += red[w][4 + 2 * k];
            }
        uint64_t* dst = a.fsums + ((size_t)b * C2w + c) * WPR;
        for (int i = 0; i < WPR; ++i) store_word(dst + i, enc_nonneg(v[i]));
    }
    // the request's last sweep workgroup (the last of them to start) draws;
    // the others are done
    if (c == C2w - 1) draw_terminal<T, MODE, PER>(a, b, cd, rs, tab);
}

// The single launch of an exact, relaxed or power call.  Its first nstream
// workgroups stream: workgroup p takes tiles p, p + nstream, ..., so the
// tiles complete about in index order, request by request, with about
// nstream tiles in flight (enough to keep HBM busy; few enough that the
// other workgroups' loads do not queue behind many microseconds of them).
// The sweep workgroups follow: every request's folding workgroups first,
// then the others, request by request; they start while the stream runs, and
// each waits only for its own request's records (and the drawing workgroup,
// the last of its request to start, for the sums of the others).  PER:
// 2048-token chunks per sweep workgroup.
template <typename T, int MODE, bool VECP, int PER>
__global__ __launch_bounds__(kThreads, kStreamWavesPerSimd) void k_single(const Args a) {
    const unsigned P = (unsigned)a.nstream, ntiles = (unsigned)(a.B * a.R * a.tpr);
    if (blockIdx.x < P) {
        for (unsigned t = blockIdx.x; t < ntiles; t += P)
            stream_tile<T, MODE, true, VECP, false, false, kTileVecs, true>(a, t);
        return;
    }
    sweep_role<T, MODE, PER>(a, (int)(blockIdx.x - P));
}

// The deciding workgroup of request b in the greedy rule's single launch:
// one lane waits for the request's last tile record, the waves fold all of
// its rows' records (waiting for any still missing), and the workgroup zeroes
// them, decides and writes the outputs.
template <typename T, bool SUM>
__device__ void greedy_role(const Args& a, const int b) {
    const int tid = threadIdx.x;
    __shared__ double tab[kExpTab];
    __shared__ RowStats rs;
    __shared__ int s_ok;
    // as in the sweep role: the last tile's record and the drafted tokens are
    // loaded while the exp table is computed
    const uint64_t* hint = a.frec + 2 * (((size_t)b * a.R + a.R - 1) * a.tpr + a.tpr - 1);
    uint64_t h = 0ull;
    if (tid == 0) h = load_word(hint);
    ChainVals cv;
    if (tid < 64) {
        chain_load_tokens<kGreedy>(a, b, cv);
        chain_load_values<T, kGreedy, false>(a, b, cv);
    }
    if (SUM) fill_exp_table(tab);
    if (tid == 0) {
        s_ok = 1;
        for (int it = 0; h == 0ull; ++it) {
            if (it >= a.spin_limit) {
                s_ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
            h = load_word(hint);
        }
    }
    __syncthreads();  // the exp table, s_ok
    if (s_ok && !fold_rows_published<kGreedy, SUM, kWaves>(a, b, a.R, rs, tab)) s_ok = 0;
    __syncthreads();
    if (!s_ok) {  // a record never arrived: report, leave the words as they are
        if (tid == 0) a.out_status[b] = 2;
        return;
    }
    // every record of the request is read: zero them for the next call
    uint64_t* w = a.frec + 2 * (size_t)b * a.R * a.tpr;
    for (int i = tid; i < 2 * a.R * a.tpr; i += kThreads) store_word(w + i, 0ull);
    greedy_finish(a, b, rs, cv);
}

// The greedy rule as one launch: nstream workgroups stream the tiles in a
// grid-stride loop and publish their records, then one deciding workgroup
// per request.  Workgroups start in index order, so a deciding workgroup
// waits only on streaming workgroups, which never wait.  NV: 16-byte loads
// per thread (8 KiB tiles for bf16 rows without log-probs).
template <typename T, bool SUM, bool VECP, int NV>
__global__ __launch_bounds__(kThreads, kStreamWavesPerSimd) void k_greedy(const Args a) {
    const unsigned P = (unsigned)a.nstream, ntiles = (unsigned)(a.B * a.R * a.tpr);
    if (blockIdx.x < P) {
        for (unsigned t = blockIdx.x; t < ntiles; t += P)
            stream_tile<T, kGreedy, SUM, VECP, false, false, NV, true>(a, t);
        return;
    }
    greedy_role<T, SUM>(a, (int)(blockIdx.x - P));
}

// Folding workgroups of the tree rule's single launch: workgroup f of
// request b folds rows kWaves*f + w (wave w), those below the request's node
// count (the stream reads no other row), and publishes their row records.
__device__ inline int tree_node_count(const Args& a, int b) {
    return min(max(a.num_nodes ? a.num_nodes[b] : a.rows_t, 1), a.rows_t);
}

template <bool SUM>
__device__ void tree_fold_role(const Args& a, const int idx) {
    const int fpr = (a.R + kWaves - 1) / kWaves;  // folding workgroups per request
    const int b = idx / fpr, f = idx - b * fpr;
    __shared__ double tab[kExpTab];
    if (SUM) {
        fill_exp_table(tab);
        __syncthreads();
    }
    const int r = f * kWaves + (int)(threadIdx.x >> 6);
    if (r < tree_node_count(a, b)) fold_publish_row<kTree, SUM>(a, b, r, tab);
}

// The deciding workgroup of request b in the tree rule's single launch: the
// node count, parents and tokens are loaded first, then the row records of
// the nodes (lane = node), which it zeroes; then the tree decision.
template <bool SUM>
__device__ void tree_decide_role(const Args& a, const int b) {
    const int tid = threadIdx.x, N = a.rows_t;
    __shared__ RowStats rs;
    __shared__ int s_ok;
    const int nraw = a.num_nodes ? a.num_nodes[b] : N;
    int p = -1, t = -1;
    if (tid >= 1 && tid < N) {
        p = a.parents[b * N + tid];
        t = a.tok[b * N + tid];
    }
    if (tid == 0) s_ok = 1;
    const int nb = min(max(nraw, 1), N);
    if (!read_row_records<kTree, SUM>(a, b, rs, nb)) s_ok = 0;
    __syncthreads();
    if (!s_ok) {  // a row record never arrived: report, leave the words as they are
        if (tid == 0) a.out_status[b] = 2;
        return;
    }
    uint64_t* w = a.frow + 2 * (size_t)b * a.R;
    for (int i = tid; i < 2 * nb; i += kThreads) store_word(w + i, 0ull);
    tree_finish<kThreads>(a, b, rs, nraw, p, t);
}

// The tree rule as one launch: one workgroup per tile streams it and
// publishes its record (nstream = the tile count), then the folding
// workgroups (kWaves rows each), then one deciding workgroup per request.  Workgroups start in index order: a
// folding workgroup waits only on streaming ones, which never wait, and a
// deciding workgroup only on folding ones.
template <typename T, bool SUM, bool VECP>
__global__ __launch_bounds__(kThreads, kStreamWavesPerSimd) void k_tree(const Args a) {
    const unsigned P = (unsigned)a.nstream;
    const unsigned nfold = (unsigned)a.B * (unsigned)((a.R + kWaves - 1) / kWaves);
    if (blockIdx.x < P) {
        // one tile per workgroup (a loop over tiles keeps more registers
        // live and spills)
        stream_tile<T, kTree, SUM, VECP, false, false, kTileVecs, true>(a, blockIdx.x);
        return;
    }
    if (blockIdx.x < P + nfold) {
        tree_fold_role<SUM>(a, (int)(blockIdx.x - P));
        return;
    }
    tree_decide_role<SUM>(a, (int)(blockIdx.x - P - nfold));
}

// The draw of sampled row g, by the row's drawing workgroup of the sampler's
// single launch.  Wave 0 waits for the row's chunk words (lane = chunk),
// rescales each chunk sum to the row max (one fp64 exp per lane), scans the
// chunks and picks the one holding u * Z; it clears the words it read.  The
// workgroup rescans that chunk, sixteen consecutive tokens per thread, with a
// block scan whose exclusive prefixes are the previous thread's inclusive
// ones bit for bit, and writes the first crossing and its log-prob.
template <typename T>
__device__ void draw_row(const Args& a, const int g) {
    constexpr int RUN = kChunk / kThreads;  // 16 tokens per thread
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
    __shared__ double tab[kExpTab];
    __shared__ int s_cstar, s_ok;
    __shared__ double s_base, s_target, s_M, s_lnZ;
    __shared__ double s_wtot[kWaves];
    __shared__ int s_pick[kWaves][3];
    fill_exp_table(tab);
    if (t == 0) s_ok = 1;
    __syncthreads();  // the exp table
    if (wave == 0) {
        const bool have = lane < a.C2;
        uint64_t* src = a.fsums + ((size_t)g * a.C2 + (have ? lane : 0)) * kRowWords;
        uint64_t w0 = 0ull, w1 = 0ull;
        bool ok = true;
        for (int it = 0;; ++it) {
            if (have) {  // both words each round, in flight together
                w0 = load_word(src);
                w1 = load_word(src + 1);
            }
            if (__ballot(have && (w0 == 0ull || w1 == 0ull)) == 0ull) break;
            if (it >= a.spin_limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (ok) {
            if (have) {  // read: zero them for the next call
                store_word(src, 0ull);
                store_word(src + 1, 0ull);
            }
            const float mc = have ? __uint_as_float((uint32_t)w1) : -INFINITY;
            const float Mr = wave_max(mc);
            // chunk record {sum of exp(l - m), m}: rescaled to the row max
            const double W = mc > -INFINITY ? dec_nonneg(w0) * exp_nonpos((double)mc - (double)Mr, tab) : 0.0;
            const double Z = wave_sum(W);
            const double target = (double)a.u[g] * Z;
            const double incl = wave_incl_scan(W);
            double excl = __shfl_up(incl, 1);
            if (lane == 0) excl = 0.0;  // [excl, incl) of consecutive chunks tile [0, Z)
            const bool hasm = have && W > 0.0;
            const unsigned long long mine = __ballot(hasm && excl <= target && target < incl);
            const unsigned long long any = __ballot(hasm);
            // the unique chunk whose interval holds target; if rounding pushed
            // target past the last boundary, the last chunk with mass
            const int cstar = mine ? __builtin_ctzll(mine) : (any ? 63 - __builtin_clzll(any) : 0);
            const double base = readlane_d(excl, cstar);
            if (lane == 0) {
                s_cstar = cstar;
                s_base = base;
                s_target = target;
                s_M = (double)Mr;
                s_lnZ = log(Z);
            }
        } else if (lane == 0) {
            s_ok = 0;
        }
    }
    __syncthreads();
    if (!s_ok) {  // a chunk's words never arrived: report, leave them as they are
        if (t == 0) a.out_status[g] = 2;
        return;
    }
    const int cstar = s_cstar;
    const double M = s_M, target = s_target;
    const T* row = reinterpret_cast<const T*>(a.T) + (size_t)g * a.V;
    const __amdgpu_buffer_rsrc_t rr = row_rsrc(row, a.V);
    const int e0 = cstar * kChunk + t * RUN;
    // weights exp(l - M) of the thread's tokens, four at a time; its sum and
    // which tokens have mass or a finite logit
    double tsum = 0.0;
    unsigned pos = 0u, fin = 0u;
#pragma unroll 1
    for (int j = 0; j < RUN; j += 4) {
        float v[4];
        Elem<T>::load4(rr, e0 + j, a.V, a.vec_t, v);
        double x[4], w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (double)v[i] - M;
        exp_nonpos_n<4>(x, w, tab);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tsum += w[i];
            pos |= (w[i] > 0.0) ? (1u << (j + i)) : 0u;
            fin |= (v[i] > -INFINITY) ? (1u << (j + i)) : 0u;
        }
    }
    const double wincl = wave_incl_scan(tsum);
    if (lane == 63) s_wtot[wave] = wincl;
    __syncthreads();
    double off = 0.0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
        if (ww < wave) off += s_wtot[ww];
    const double tincl = wincl + off;
    double texcl = __shfl_up(tincl, 1);
    if (lane == 0) texcl = off;
    // first crossing of the running sum past target in this thread's tokens
    // (read again, now from cache, and their weights formed again, bit for
    // bit).  Threads whose interval ends at or before target have none; a
    // thread past it crosses at its first token with mass, which covers a
    // rounding that leaves the crossing just past the interval holding target.
    int cand = INT_MAX;
    if (target < s_base + tincl) {
        double cum = s_base + texcl;
#pragma unroll 1
        for (int j = 0; j < RUN && cand == INT_MAX; j += 4) {
            float v[4];
            Elem<T>::load4(rr, e0 + j, a.V, a.vec_t, v);
            double x[4], w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (double)v[i] - M;
            exp_nonpos_n<4>(x, w, tab);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (w[i] > 0.0 && cand == INT_MAX) {
                    cum += w[i];
                    if (cum > target) cand = e0 + j + i;
                }
            }
        }
    }
    const int lastpos = pos ? e0 + 31 - __builtin_clz(pos) : -1;
    const int anypos = fin ? e0 + 31 - __builtin_clz(fin) : -1;
    const int wc = wave_min_i(cand), wl = wave_max_i(lastpos), wa = wave_max_i(anypos);
    if (lane == 0) {
        s_pick[wave][0] = wc;
        s_pick[wave][1] = wl;
        s_pick[wave][2] = wa;
    }
    __syncthreads();
    int yc = INT_MAX, yl = -1, ya = -1;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
        yc = min(yc, s_pick[ww][0]);
        yl = max(yl, s_pick[ww][1]);
        ya = max(ya, s_pick[ww][2]);
    }
    // The crossing token; if rounding left none, the last token with mass in
    // the chunk; if the chunk had none, its last finite token.  Always a valid
    // index.
    int y = (yc != INT_MAX) ? yc : (yl >= 0 ? yl : ya);
    if (y < 0 || y >= a.V) y = 0;
    if (t == 0) {
        const float ly = Elem<T>::at(row, (size_t)y);
        a.out_tok[g] = y;
        if (a.out_tlp) a.out_tlp[g] = (float)(((double)ly - M) - s_lnZ);
        a.out_status[g] = 0;
    }
}

// The draft sampler as one launch: rows x tpr streaming workgroups (one tile
// each, chunk records published), then one drawing workgroup per row.
// Workgroups start in index order, so a drawing workgroup waits only on
// streaming workgroups, which never wait.
template <typename T, bool VECP>
__global__ __launch_bounds__(kThreads, kStreamWavesPerSimd) void k_sample_rows(const Args a) {
    const unsigned ns = (unsigned)a.B * (unsigned)a.tpr;
    if (blockIdx.x < ns) {
        rows_tile<T, VECP>(a, blockIdx.x);
        return;
    }
    draw_row<T>(a, (int)(blockIdx.x - ns));
}

// ------------------------------------------------------------------- host
inline int esize(spec_dtype dt) { return dt == SPEC_BF16 ? 2 : 4; }

// Compute units of the current device, looked up once per device (256 if the
// lookup fails); a single launch streams with kStreamPerCu workgroups per
// compute unit.
constexpr int kStreamPerCu = 8;
constexpr int kStreamPerCuBig = 6;  // single launches whose sweep workgroups outnumber the streamers
constexpr int kMaxCuCache = 64;
std::atomic<int> g_cus[kMaxCuCache];
inline int compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    if (dev >= 0 && dev < kMaxCuCache) cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        if (dev >= 0 && dev < kMaxCuCache) g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}
inline int stream_workgroups() { return kStreamPerCu * compute_units(); }
// Streaming workgroups of the greedy and tree launches: one per tile
// (measured faster than a grid-stride loop for the greedy rule at these
// sizes), up to a cap that keeps the grid far below 2^32 threads; above it
// they loop.
constexpr int kMaxStreamGroups = 1 << 20;
inline int tile_elems(spec_dtype dt) { return kTileBytes / esize(dt); }
inline int tpr_of(spec_dtype dt, int V) { return (V + tile_elems(dt) - 1) / tile_elems(dt); }
constexpr int kSmallTileElems = kThreads * kSmallTileVecs * 8;  // bf16 elements of an 8 KiB tile
// Tiles per row of the stream (8 KiB tiles have as many as an fp32 row's 16
// KiB tiles, so the workspace query, sized for fp32, covers them).
inline int stream_tpr(spec_dtype dt, int V, bool small) {
    return small ? (V + kSmallTileElems - 1) / kSmallTileElems : tpr_of(dt, V);
}
inline int c2_of(spec_dtype, int V) { return (V + kChunk - 1) / kChunk; }

inline bool vec_ok(const void* p, spec_dtype dt, int V) {
    return ((uintptr_t)p % 16 == 0) && (((size_t)V * esize(dt)) % 16 == 0);
}

spec_status check_ws(void* ws, size_t bytes, int B, int R, int V, spec_dtype dt, bool small = false) {
    if (!ws || ((uintptr_t)ws % 256) != 0) return SPEC_EWORKSPACE;
    const Layout L = make_layout(B, R, stream_tpr(dt, V, small), c2_of(dt, V));
    return bytes >= L.total ? SPEC_OK : SPEC_EWORKSPACE;
}

// Bound of the single launches' waits (spec_set_spin_limit).
std::atomic<int> g_spin_limit{kSpinLimit};

// One-shot profiling hook: events for the kernels of the next call made from
// this thread.
thread_local hipEvent_t g_prof[3] = {nullptr, nullptr, nullptr};

// The streaming kernel over B * R rows of a.V logits, with the dispatch's
// own start and stop events when given.
// NV: 16-byte loads per thread, kTileVecs (16 KiB tiles) or kSmallTileVecs
// (8 KiB tiles, bf16 only); a.tpr must match it.
template <int MODE, bool SUM, bool XV, bool SHARD = false, int NV = kTileVecs>
spec_status launch_stream(const Args& a, spec_dtype dt, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid((unsigned)a.B * (unsigned)a.R * (unsigned)a.tpr), block(kThreads);
    const bool vecp = a.vec_t && (!uses_draft(MODE) || a.vec_d);
    if (dt == SPEC_BF16) {
        if (vecp)
            hipExtLaunchKernelGGL((k_stream<uint16_t, MODE, SUM, true, XV, SHARD, NV>), grid, block, 0, st, e0, e1, 0, a);
        else
            hipExtLaunchKernelGGL((k_stream<uint16_t, MODE, SUM, false, XV, SHARD, NV>), grid, block, 0, st, e0, e1, 0, a);
    } else if constexpr (NV == kTileVecs) {
        if (vecp)
            hipExtLaunchKernelGGL((k_stream<float, MODE, SUM, true, XV, SHARD, NV>), grid, block, 0, st, e0, e1, 0, a);
        else
            hipExtLaunchKernelGGL((k_stream<float, MODE, SUM, false, XV, SHARD, NV>), grid, block, 0, st, e0, e1, 0, a);
    } else {
        return SPEC_EINVAL;  // small tiles are bf16 only (never chosen for fp32)
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

// Takes the one-shot profiling events, clearing them.
inline void take_prof(hipEvent_t (&ev)[3]) {
    for (int i = 0; i < 3; ++i) {
        ev[i] = g_prof[i];
        g_prof[i] = nullptr;
    }
}

// The tree rule's single launch (k_tree): one streaming workgroup per tile,
// the folding workgroups, one deciding workgroup per request (tree_grid_ok
// bounds the grid).  With the profiling hook set, the launch carries the start and
// stop events.
template <bool SUM>
spec_status launch_tree(Args a, spec_dtype dt, hipStream_t st) {
    a.tpr = tpr_of(dt, a.V);
    a.Vtot = a.V;
    const Layout lay = make_layout(a.B, a.R, a.tpr, a.C2);
    a.frec = reinterpret_cast<uint64_t*>(a.ws + lay.frec);
    a.frow = reinterpret_cast<uint64_t*>(a.ws + lay.frow);
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    a.nstream = a.B * a.R * a.tpr;
    const unsigned nfold = (unsigned)a.B * (unsigned)((a.R + kWaves - 1) / kWaves);
    const dim3 grid((unsigned)a.nstream + nfold + (unsigned)a.B), block(kThreads);
    hipEvent_t ev[3];
    take_prof(ev);
    if (dt == SPEC_BF16) {
        if (a.vec_t)
            hipExtLaunchKernelGGL((k_tree<uint16_t, SUM, true>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else
            hipExtLaunchKernelGGL((k_tree<uint16_t, SUM, false>), grid, block, 0, st, ev[0], ev[1], 0, a);
    } else {
        if (a.vec_t)
            hipExtLaunchKernelGGL((k_tree<float, SUM, true>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else
            hipExtLaunchKernelGGL((k_tree<float, SUM, false>), grid, block, 0, st, ev[0], ev[1], 0, a);
    }
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

// The single launch of an exact, relaxed or power call (k_single): the
// streaming workgroups, then one sweep workgroup per (request, chunk).  With
// the profiling hook set, the launch carries the start and stop events: the
// whole call is this one kernel.
template <int MODE>
spec_status launch_single(Args a, spec_dtype dt, hipStream_t st) {
    a.tpr = tpr_of(dt, a.V);
    a.Vtot = a.V;
    const Layout lay = make_layout(a.B, a.R, a.tpr, a.C2);
    a.frec = reinterpret_cast<uint64_t*>(a.ws + lay.frec);
    a.fsums = reinterpret_cast<uint64_t*>(a.ws + lay.fsums);
    a.frow = reinterpret_cast<uint64_t*>(a.ws + lay.frow);
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    const bool vecp = a.vec_t && (!uses_draft(MODE) || a.vec_d);
    // Aligned bf16 rows take one sweep workgroup per 2048-token record when
    // the chip holds them all at once beside the streamers' slots (measured
    // faster at B=32, V=128256); otherwise, and on the other paths, one per
    // two records (twice the workgroups was slower at B=64, V=151936).  When
    // they would not all fit, 6 streaming workgroups per compute unit leave
    // two slots per unit to sweep workgroups during the stream (measured at
    // B=64, K=8, V=151936: exact 75.3 -> 74.3 us, relaxed 44.3 -> 43.8; at
    // B=32, V=128256 it made no difference to exact and slowed power).
    a.C2s = (a.V + kSweepChunk - 1) / kSweepChunk;
    const bool big = (long long)a.B * a.C2s > stream_workgroups();
    a.nstream = min(a.B * a.R * a.tpr, big ? kStreamPerCuBig * compute_units() : stream_workgroups());
    const bool per1 = dt == SPEC_BF16 && vecp && !big;
    const int C2w = per1 ? a.C2s : (a.C2s + kSweepSplit - 1) / kSweepSplit;
    const dim3 grid((unsigned)a.nstream + (unsigned)a.B * (unsigned)C2w), block(kThreads);
    hipEvent_t ev[3];
    take_prof(ev);
    if (dt == SPEC_BF16) {
        if (per1)
            hipExtLaunchKernelGGL((k_single<uint16_t, MODE, true, 1>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else if (vecp)
            hipExtLaunchKernelGGL((k_single<uint16_t, MODE, true, 2>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else
            hipExtLaunchKernelGGL((k_single<uint16_t, MODE, false, 2>), grid, block, 0, st, ev[0], ev[1], 0, a);
    } else {
        if (vecp)
            hipExtLaunchKernelGGL((k_single<float, MODE, true, 2>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else
            hipExtLaunchKernelGGL((k_single<float, MODE, false, 2>), grid, block, 0, st, ev[0], ev[1], 0, a);
    }
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

// Whether the greedy rule's single launch streams 8 KiB tiles: bf16 rows
// without log-probs, when 16 KiB tiles would number fewer than the streaming
// workgroups the chip holds at once (measured: 8 KiB tiles are faster at
// B=8, K=5, V=128256 and slower at B=32).
inline bool greedy_small_tiles(spec_dtype dt, int V, long long rows, bool logprobs) {
    return !logprobs && dt == SPEC_BF16 && rows * tpr_of(dt, V) < stream_workgroups();
}

template <typename T, bool SUM, int NV>
void launch_greedy_kernel(const Args& a, bool vecp, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    if (vecp)
        hipExtLaunchKernelGGL((k_greedy<T, SUM, true, NV>), grid, dim3(kThreads), 0, st, e0, e1, 0, a);
    else
        hipExtLaunchKernelGGL((k_greedy<T, SUM, false, NV>), grid, dim3(kThreads), 0, st, e0, e1, 0, a);
}

// The greedy rule's single launch (k_greedy): the streaming workgroups, then
// one deciding workgroup per request.  With the profiling hook set, the
// launch carries the start and stop events.
template <bool SUM>
spec_status launch_greedy(Args a, spec_dtype dt, hipStream_t st) {
    const bool small = greedy_small_tiles(dt, a.V, (long long)a.B * a.R, SUM);
    a.tpr = stream_tpr(dt, a.V, small);
    a.Vtot = a.V;
    const Layout lay = make_layout(a.B, a.R, a.tpr, a.C2);
    a.frec = reinterpret_cast<uint64_t*>(a.ws + lay.frec);
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    a.nstream = (int)min((long long)a.B * a.R * a.tpr, (long long)kMaxStreamGroups);
    const dim3 grid((unsigned)a.nstream + (unsigned)a.B);
    hipEvent_t ev[3];
    take_prof(ev);
    if (dt != SPEC_BF16)
        launch_greedy_kernel<float, SUM, kTileVecs>(a, a.vec_t, grid, st, ev[0], ev[1]);
    else if (!SUM && small)  // 8 KiB tiles (never with log-probs)
        launch_greedy_kernel<uint16_t, false, kSmallTileVecs>(a, a.vec_t, grid, st, ev[0], ev[1]);
    else
        launch_greedy_kernel<uint16_t, SUM, kTileVecs>(a, a.vec_t, grid, st, ev[0], ev[1]);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

// The tree launch's grid (one workgroup per tile, the folding workgroups,
// one deciding workgroup per request) stays below 2^32 threads.
inline bool tree_grid_ok(spec_dtype dt, int B, int N, int V) {
    const long long wg = (long long)B * N * tpr_of(dt, V) + (long long)B * ((N + kWaves - 1) / kWaves) + B;
    return wg * kThreads < (1ll << 32);
}

// The single launch's grid (streaming tiles plus one sweep workgroup per
// chunk) stays below 2^32 threads.
inline bool single_grid_ok(spec_dtype dt, int B, int R, int V) {
    const long long wg = (long long)B * R * tpr_of(dt, V) + (long long)B * c2_of(dt, V);
    return wg * kThreads < (1ll << 32);
}

// ------------------------------------------------------ vocabulary shards
// One shard's record slot: the tile records of its B * R rows, then the
// drafted-token logits ([B][K][2] floats, sized [B][R][2]).
struct ShardLayout {
    size_t xv, slot;
};
inline ShardLayout shard_layout(spec_dtype dt, int B, int R, int Vs) {
    ShardLayout L;
    L.xv = align_up((size_t)B * R * tpr_of(dt, Vs) * sizeof(Seg), 256);
    L.slot = align_up(L.xv + (size_t)B * R * 2 * sizeof(float), 256);
    return L;
}
inline size_t shard_sums_slot(int B, int Vs) { return align_up((size_t)B * c2_of(SPEC_F32, Vs) * sizeof(ChunkSums), 256); }
inline size_t shard_ws_bytes(int B) { return align_up((size_t)B * 64, 256); }

bool sizes_ok(spec_dtype dt, int B, int K, int V, long rows_per_req);

// Shard count, shard index and the one-wave limits of the combine and the
// sample scan.
bool shard_ok(spec_dtype dt, int B, int K, int V, int G, int shard, long rows) {
    if (G < 1 || V < 1 || V % G != 0 || shard < 0 || shard >= G) return false;
    if (!sizes_ok(dt, B, K, V, rows)) return false;
    const int Vs = V / G;
    return (long)G * tpr_of(dt, Vs) <= 64 && (long)G * c2_of(dt, Vs) <= 64;
}

inline bool buf_ok(const void* p, size_t bytes, size_t need) {
    return p && ((uintptr_t)p % 256) == 0 && bytes >= need;
}

// G gathered slots of `slot` bytes each (slot 0 for invalid sizes).
inline bool gathered_ok(const void* p, size_t bytes, int G, size_t slot) {
    return slot > 0 && G >= 1 && buf_ok(p, bytes, (size_t)G * slot);
}

// Shard-local argument block: V is the shard's column count, Vtot the
// vocabulary.
inline Args shard_args(spec_dtype dt, int B, int K, int V, int G, int shard, int rows_t, int R) {
    Args a = {};
    a.B = B;
    a.K = K;
    a.V = V / G;
    a.Vtot = V;
    a.G = G;
    a.shard = shard;
    a.rows_t = rows_t;
    a.R = R;
    a.tpr = tpr_of(dt, a.V);
    a.C2 = c2_of(dt, a.V);
    a.L = rows_t;
    return a;
}

// Points the combine at the G gathered record slots.
inline void gathered_records(Args& a, spec_dtype dt, const void* records) {
    const ShardLayout L = shard_layout(dt, a.B, a.R, a.V);
    a.segs = reinterpret_cast<Seg*>(const_cast<void*>(records));
    a.slot_segs = L.slot / sizeof(Seg);
    a.xv_in = reinterpret_cast<const float*>(static_cast<const unsigned char*>(records) + L.xv);
    a.slot_xv = L.slot / sizeof(float);
}

template <int MODE, bool SUM>
spec_status shard_stats(Args a, spec_dtype dt, void* out_record, hipStream_t st) {
    const ShardLayout L = shard_layout(dt, a.B, a.R, a.V);
    a.segs = reinterpret_cast<Seg*>(out_record);
    a.xv_out = reinterpret_cast<float*>(static_cast<unsigned char*>(out_record) + L.xv);
    hipEvent_t ev[3];
    take_prof(ev);
    constexpr bool XV = uses_draft(MODE) || MODE == kRelaxed;
    if (launch_stream<MODE, SUM, XV, MODE == kRelaxed>(a, dt, st, ev[0], ev[1]) != SPEC_OK) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

// One per-request kernel of a sharded step, with the profiling events around
// its dispatch when set.
template <typename K>
spec_status shard_launch(K kernel, dim3 grid, dim3 block, const Args& a, hipStream_t st) {
    hipEvent_t ev[3];
    take_prof(ev);
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev[0], ev[1], 0, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

// A caller written in C may pass any int as the dtype (a C enum is an int);
// in C++ reading a value outside the enumerators through the enum type is
// undefined, so the argument's bytes are inspected before it is ever read as
// spec_dtype.
static_assert(sizeof(spec_dtype) == sizeof(int), "spec_dtype is passed as an int");
bool dtype_ok(const spec_dtype& dt) {
    int v;
    memcpy(&v, &dt, sizeof v);
    return v == SPEC_F32 || v == SPEC_BF16;
}

// The draft sampler's workspace: the layout of one row per request (it uses
// the chunk-sum region) and a row-count tail that the size query has always
// included.
size_t sample_layout_bytes(int rows, int V, spec_dtype dt) {
    return make_layout(rows, 1, tpr_of(dt, V), c2_of(dt, V)).total;
}

bool sizes_ok(spec_dtype dt, int B, int K, int V, long rows_per_req) {
    if (B < 1 || B > kMaxB || K < 1 || V < 1 || V > SPEC_MAX_V) return false;
    if (rows_per_req < 1 || rows_per_req > kMaxRows) return false;
    // The streaming grid's size in threads is a 32-bit quantity: one 16 KiB
    // tile per workgroup of kThreads, so at most 2^24 tiles (256 GiB of
    // logits) per call.  Element offsets stay far inside 64 bits.
    const long long tiles = (long long)B * rows_per_req * tpr_of(dt, V);
    return tiles * kThreads < (1ll << 32) && (long long)B * rows_per_req * V < (1ll << 40);
}

}  // namespace

// ============================================================== C interface
extern "C" {

size_t spec_verify_workspace_bytes(int B, int rows_per_request, int V) {
    if (B < 1 || B > kMaxB || rows_per_request < 1 || rows_per_request > kMaxRows || V < 1 ||
        V > SPEC_MAX_V)
        return 0;
    // fp32 has the most tiles per row, so its layout bounds both dtypes
    const Layout L = make_layout(B, rows_per_request, tpr_of(SPEC_F32, V), c2_of(SPEC_F32, V));
    return L.total;
}

void spec_verify_profile_next_call(void* before_stream, void* after_stream, void* after_call) {
    g_prof[0] = static_cast<hipEvent_t>(before_stream);
    g_prof[1] = static_cast<hipEvent_t>(after_stream);
    g_prof[2] = static_cast<hipEvent_t>(after_call);
}

void spec_set_spin_limit(int limit) {
    g_spin_limit.store(limit < 0 ? kSpinLimit : limit, std::memory_order_relaxed);
}

const char* spec_status_string(int s) {
    switch (s) {
        case SPEC_OK: return "ok";
        case SPEC_EINVAL: return "invalid argument";
        case SPEC_EDTYPE: return "unsupported dtype";
        case SPEC_EWORKSPACE: return "workspace missing, misaligned or too small";
        case SPEC_EHIP: return "HIP launch failed";
        case SPEC_ESCRATCH: return "call needs more than the static scratch array holds";
        default: return "unknown status";
    }
}

spec_status spec_verify_greedy(const void* target_logits, spec_dtype dtype,
                               const int32_t* draft_tokens, int B, int K, int V,
                               int32_t* out_tokens, int32_t* out_accept_len,
                               float* out_target_logprob, float* out_behavior_logprob,
                               int32_t* out_status, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(dtype, B, K, V, K + 1)) return SPEC_EINVAL;
    if (!target_logits || !draft_tokens || !out_tokens || !out_accept_len || !out_status)
        return SPEC_EINVAL;
    const spec_status ws = check_ws(workspace, workspace_bytes, B, K + 1, V, dtype,
                                    greedy_small_tiles(dtype, V, (long long)B * (K + 1), out_target_logprob));
    if (ws != SPEC_OK) return ws;
    Args a = {};
    a.T = target_logits;
    a.tok = draft_tokens;
    a.B = B;
    a.K = K;
    a.V = V;
    a.rows_t = K + 1;
    a.R = K + 1;
    a.C2 = c2_of(dtype, V);
    a.vec_t = vec_ok(target_logits, dtype, V);
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    a.L = K + 1;
    a.ws = static_cast<unsigned char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (out_target_logprob) return launch_greedy<true>(a, dtype, st);
    return launch_greedy<false>(a, dtype, st);
}

spec_status spec_verify_exact(const void* target_logits, const void* draft_logits,
                              spec_dtype dtype, const int32_t* draft_tokens, const float* uniforms,
                              int B, int K, int V, int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_target_logprob, float* out_behavior_logprob,
                              int32_t* out_status, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(dtype, B, K, V, 2 * K + 1) || !single_grid_ok(dtype, B, 2 * K + 1, V))
        return SPEC_EINVAL;
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !out_tokens ||
        !out_accept_len || !out_status)
        return SPEC_EINVAL;
    const spec_status ws = check_ws(workspace, workspace_bytes, B, 2 * K + 1, V, dtype);
    if (ws != SPEC_OK) return ws;
    Args a = {};
    a.T = target_logits;
    a.D = draft_logits;
    a.tok = draft_tokens;
    a.u = uniforms;
    a.B = B;
    a.K = K;
    a.V = V;
    a.rows_t = K + 1;
    a.R = 2 * K + 1;
    a.C2 = c2_of(dtype, V);
    a.vec_t = vec_ok(target_logits, dtype, V);
    a.vec_d = vec_ok(draft_logits, dtype, V);
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    a.L = K + 1;
    a.ws = static_cast<unsigned char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return launch_single<kExact>(a, dtype, st);
}

spec_status spec_verify_relaxed(const void* target_logits, spec_dtype dtype,
                                const int32_t* draft_tokens, const float* uniforms, int B, int K,
                                int V, float tau, int top_k, int32_t* out_tokens,
                                int32_t* out_accept_len, float* out_target_logprob,
                                float* out_behavior_logprob, int32_t* out_status, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(dtype, B, K, V, K + 1) || !single_grid_ok(dtype, B, K + 1, V))
        return SPEC_EINVAL;
    if (tau != tau || top_k < 0) return SPEC_EINVAL;
    if (!target_logits || !draft_tokens || !uniforms || !out_tokens || !out_accept_len ||
        !out_status)
        return SPEC_EINVAL;
    const spec_status ws = check_ws(workspace, workspace_bytes, B, K + 1, V, dtype);
    if (ws != SPEC_OK) return ws;
    Args a = {};
    a.T = target_logits;
    a.tok = draft_tokens;
    a.u = uniforms;
    a.B = B;
    a.K = K;
    a.V = V;
    a.rows_t = K + 1;
    a.R = K + 1;
    a.C2 = c2_of(dtype, V);
    a.vec_t = vec_ok(target_logits, dtype, V);
    a.tau = tau;
    a.top_k = top_k;
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    a.L = K + 1;
    a.ws = static_cast<unsigned char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return launch_single<kRelaxed>(a, dtype, st);
}

spec_status spec_verify_power(const void* target_logits, const void* draft_logits,
                              spec_dtype dtype, const int32_t* draft_tokens, const float* uniforms,
                              int B, int K, int V, float alpha, int32_t* out_tokens,
                              int32_t* out_accept_len, float* out_target_logprob,
                              float* out_behavior_logprob, int32_t* out_status, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(dtype, B, K, V, 2 * K + 1) || !single_grid_ok(dtype, B, 2 * K + 1, V))
        return SPEC_EINVAL;
    if (!(alpha >= 0.f) || alpha == INFINITY) return SPEC_EINVAL;
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !out_tokens ||
        !out_accept_len || !out_status)
        return SPEC_EINVAL;
    const spec_status ws = check_ws(workspace, workspace_bytes, B, 2 * K + 1, V, dtype);
    if (ws != SPEC_OK) return ws;
    Args a = {};
    a.T = target_logits;
    a.D = draft_logits;
    a.tok = draft_tokens;
    a.u = uniforms;
    a.B = B;
    a.K = K;
    a.V = V;
    a.rows_t = K + 1;
    a.R = 2 * K + 1;
    a.C2 = c2_of(dtype, V);
    a.vec_t = vec_ok(target_logits, dtype, V);
    a.vec_d = vec_ok(draft_logits, dtype, V);
    a.alpha = alpha;
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    a.L = K + 1;
    a.ws = static_cast<unsigned char*>(workspace);
    return launch_single<kPower>(a, dtype, static_cast<hipStream_t>(stream));
}

size_t spec_sample_workspace_bytes(int rows, int V) {
    if (rows < 1 || rows > kMaxB || V < 1 || V > SPEC_MAX_V) return 0;
    return sample_layout_bytes(rows, V, SPEC_F32);  // fp32 bounds both dtypes
}

spec_status spec_sample_drafts(const void* logits, spec_dtype dtype, const float* uniforms,
                               int rows, int V, int32_t* out_tokens, float* out_logprob,
                               int32_t* out_status, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (rows < 1 || rows > kMaxB || V < 1 || V > SPEC_MAX_V) return SPEC_EINVAL;
    if (!logits || !uniforms || !out_tokens || !out_status) return SPEC_EINVAL;
    if (!workspace || ((uintptr_t)workspace % 256) != 0 ||
        workspace_bytes < sample_layout_bytes(rows, V, dtype))
        return SPEC_EWORKSPACE;
    Args a = {};
    a.T = logits;
    a.u = uniforms;
    a.B = rows;
    a.K = 0;
    a.V = V;
    a.rows_t = 1;
    a.R = 1;
    a.C2 = c2_of(dtype, V);
    a.vec_t = vec_ok(logits, dtype, V);
    a.tau = 2.f;  // unused: there is no draft to test
    a.top_k = 0;
    a.out_tok = out_tokens;
    a.out_tlp = out_logprob;
    a.out_status = out_status;
    a.L = 1;
    a.ws = static_cast<unsigned char*>(workspace);
    a.tpr = tpr_of(dtype, V);
    a.Vtot = V;
    a.fsums = reinterpret_cast<uint64_t*>(a.ws + make_layout(rows, 1, a.tpr, a.C2).fsums);
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    // one launch: the tiles publish fp64 chunk sums, each row's drawing
    // workgroup picks them up and draws
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t ev[3];
    take_prof(ev);
    const dim3 grid((unsigned)rows * (unsigned)a.tpr + (unsigned)rows), block(kThreads);
    if (dtype == SPEC_BF16) {
        if (a.vec_t)
            hipExtLaunchKernelGGL((k_sample_rows<uint16_t, true>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else
            hipExtLaunchKernelGGL((k_sample_rows<uint16_t, false>), grid, block, 0, st, ev[0], ev[1], 0, a);
    } else {
        if (a.vec_t)
            hipExtLaunchKernelGGL((k_sample_rows<float, true>), grid, block, 0, st, ev[0], ev[1], 0, a);
        else
            hipExtLaunchKernelGGL((k_sample_rows<float, false>), grid, block, 0, st, ev[0], ev[1], 0, a);
    }
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

spec_status spec_verify_tree(const void* target_logits, spec_dtype dtype,
                             const int32_t* node_tokens, const int32_t* parents,
                             const int32_t* num_nodes, int B, int N, int V,
                             int32_t* out_path_nodes, int32_t* out_tokens, int32_t* out_accept_len,
                             float* out_target_logprob, float* out_behavior_logprob,
                             int32_t* out_status, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (N < 1 || N > SPEC_MAX_NODES || !sizes_ok(dtype, B, 1, V, N) || !tree_grid_ok(dtype, B, N, V))
        return SPEC_EINVAL;
    if (!target_logits || !node_tokens || !parents || !out_path_nodes || !out_tokens ||
        !out_accept_len || !out_status)
        return SPEC_EINVAL;
    const spec_status ws = check_ws(workspace, workspace_bytes, B, N, V, dtype);
    if (ws != SPEC_OK) return ws;
    Args a = {};
    a.T = target_logits;
    a.tok = node_tokens;
    a.parents = parents;
    a.num_nodes = num_nodes;
    a.B = B;
    a.K = 0;
    a.V = V;
    a.rows_t = N;
    a.R = N;
    a.C2 = c2_of(dtype, V);
    a.vec_t = vec_ok(target_logits, dtype, V);
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    a.out_path = out_path_nodes;
    a.L = N;
    a.ws = static_cast<unsigned char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (out_target_logprob) return launch_tree<true>(a, dtype, st);
    return launch_tree<false>(a, dtype, st);
}

size_t spec_read_ceiling_out_words(size_t bytes) {
    if (bytes < 16 || bytes % 16 != 0) return 0;
    return (bytes + kTileBytes - 1) / kTileBytes;
}

spec_status spec_read_ceiling(const void* data, size_t bytes, uint32_t* out, void* stream) {
    const size_t words = spec_read_ceiling_out_words(bytes);
    if (!data || !out || words == 0 || words > (size_t)INT_MAX || ((uintptr_t)data % 16) != 0)
        return SPEC_EINVAL;
    hipEvent_t ev[3];
    take_prof(ev);
    hipExtLaunchKernelGGL(k_read, dim3((unsigned)words), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                          ev[0], ev[1], 0, static_cast<const unsigned char*>(data), bytes / 16, out);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (ev[2] && hipEventRecord(ev[2], static_cast<hipStream_t>(stream)) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

// ------------------------------------------------------ vocabulary shards
size_t spec_shard_record_bytes(spec_dtype dtype, int B, int rows_per_request, int V, int G) {
    if (!dtype_ok(dtype) || !shard_ok(dtype, B, 1, V, G, 0, rows_per_request)) return 0;
    return shard_layout(dtype, B, rows_per_request, V / G).slot;
}

size_t spec_shard_sums_bytes(int B, int V, int G) {
    if (B < 1 || B > kMaxB || G < 1 || V < 1 || V > SPEC_MAX_V || V % G != 0) return 0;
    return shard_sums_slot(B, V / G);
}

size_t spec_shard_workspace_bytes(int B) {
    if (B < 1 || B > kMaxB) return 0;
    return shard_ws_bytes(B);
}

spec_status spec_shard_stats_greedy(const void* target_shard, spec_dtype dtype, int B, int K,
                                    int V, int G, int shard, int logprobs, void* out_record,
                                    size_t record_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, shard, K + 1) || !target_shard)
        return SPEC_EINVAL;
    Args a = shard_args(dtype, B, K, V, G, shard, K + 1, K + 1);
    if (!buf_ok(out_record, record_bytes, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    a.T = target_shard;
    a.vec_t = vec_ok(target_shard, dtype, a.V);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (logprobs) return shard_stats<kGreedy, true>(a, dtype, out_record, st);
    return shard_stats<kGreedy, false>(a, dtype, out_record, st);
}

spec_status spec_shard_stats_tree(const void* target_shard, spec_dtype dtype,
                                  const int32_t* num_nodes, int B, int N, int V, int G, int shard,
                                  int logprobs, void* out_record, size_t record_bytes,
                                  void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (N < 1 || N > SPEC_MAX_NODES || !shard_ok(dtype, B, 1, V, G, shard, N) || !target_shard)
        return SPEC_EINVAL;
    Args a = shard_args(dtype, B, 0, V, G, shard, N, N);
    if (!buf_ok(out_record, record_bytes, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    a.T = target_shard;
    a.num_nodes = num_nodes;
    a.vec_t = vec_ok(target_shard, dtype, a.V);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (logprobs) return shard_stats<kTree, true>(a, dtype, out_record, st);
    return shard_stats<kTree, false>(a, dtype, out_record, st);
}

spec_status spec_shard_stats_exact(const void* target_shard, const void* draft_shard,
                                   spec_dtype dtype, const int32_t* draft_tokens, int B, int K,
                                   int V, int G, int shard, void* out_record, size_t record_bytes,
                                   void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, shard, 2 * K + 1)) return SPEC_EINVAL;
    if (!target_shard || !draft_shard || !draft_tokens) return SPEC_EINVAL;
    Args a = shard_args(dtype, B, K, V, G, shard, K + 1, 2 * K + 1);
    if (!buf_ok(out_record, record_bytes, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    a.T = target_shard;
    a.D = draft_shard;
    a.tok = draft_tokens;
    a.vec_t = vec_ok(target_shard, dtype, a.V);
    a.vec_d = vec_ok(draft_shard, dtype, a.V);
    return shard_stats<kExact, true>(a, dtype, out_record, static_cast<hipStream_t>(stream));
}

spec_status spec_shard_combine_greedy(const void* records, size_t records_bytes, spec_dtype dtype,
                                      const int32_t* draft_tokens, int B, int K, int V, int G,
                                      int32_t* out_tokens, int32_t* out_accept_len,
                                      float* out_target_logprob, float* out_behavior_logprob,
                                      int32_t* out_status, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, 0, K + 1)) return SPEC_EINVAL;
    Args a = shard_args(dtype, B, K, V, G, 0, K + 1, K + 1);
    if (!gathered_ok(records, records_bytes, G, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    if (!draft_tokens || !out_tokens || !out_accept_len || !out_status) return SPEC_EINVAL;
    gathered_records(a, dtype, records);
    a.tok = draft_tokens;
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(B), block(decide_threads(kGreedy));
    if (dtype == SPEC_BF16) {
        if (out_target_logprob) return shard_launch(k_decide<uint16_t, kGreedy, true, true>, grid, block, a, st);
        return shard_launch(k_decide<uint16_t, kGreedy, false, true>, grid, block, a, st);
    }
    if (out_target_logprob) return shard_launch(k_decide<float, kGreedy, true, true>, grid, block, a, st);
    return shard_launch(k_decide<float, kGreedy, false, true>, grid, block, a, st);
}

spec_status spec_shard_combine_tree(const void* records, size_t records_bytes, spec_dtype dtype,
                                    const int32_t* node_tokens, const int32_t* parents,
                                    const int32_t* num_nodes, int B, int N, int V, int G,
                                    int32_t* out_path_nodes, int32_t* out_tokens,
                                    int32_t* out_accept_len, float* out_target_logprob,
                                    float* out_behavior_logprob, int32_t* out_status,
                                    void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (N < 1 || N > SPEC_MAX_NODES || !shard_ok(dtype, B, 1, V, G, 0, N)) return SPEC_EINVAL;
    Args a = shard_args(dtype, B, 0, V, G, 0, N, N);
    if (!gathered_ok(records, records_bytes, G, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    if (!node_tokens || !parents || !out_path_nodes || !out_tokens || !out_accept_len || !out_status)
        return SPEC_EINVAL;
    gathered_records(a, dtype, records);
    a.tok = node_tokens;
    a.parents = parents;
    a.num_nodes = num_nodes;
    a.out_path = out_path_nodes;
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(B), block(kDecideThreads);
    if (dtype == SPEC_BF16) {
        if (out_target_logprob) return shard_launch(k_decide<uint16_t, kTree, true, true>, grid, block, a, st);
        return shard_launch(k_decide<uint16_t, kTree, false, true>, grid, block, a, st);
    }
    if (out_target_logprob) return shard_launch(k_decide<float, kTree, true, true>, grid, block, a, st);
    return shard_launch(k_decide<float, kTree, false, true>, grid, block, a, st);
}

}  // extern "C"

namespace {

// Rows per request of a chain rule: target K+1, plus draft K for the rules
// that test p/q.
constexpr int chain_rows(int mode, int K) { return uses_draft(mode) ? 2 * K + 1 : K + 1; }

template <int MODE>
spec_status shard_sweep(const void* target_shard, const void* draft_shard, spec_dtype dtype,
                        const void* records, size_t records_bytes, const int32_t* draft_tokens, const float* uniforms,
                        int B, int K, int V, int G, int shard, float alpha, float tau, int top_k,
                        int32_t* out_tokens, int32_t* out_accept_len, float* out_target_logprob,
                        float* out_behavior_logprob, int32_t* out_status, void* out_sums,
                        size_t sums_bytes, void* workspace, size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, shard, chain_rows(MODE, K))) return SPEC_EINVAL;
    if (MODE == kPower && (!(alpha >= 0.f) || alpha == INFINITY)) return SPEC_EINVAL;
    if (MODE == kRelaxed && (tau != tau || top_k < 0)) return SPEC_EINVAL;
    Args a = shard_args(dtype, B, K, V, G, shard, K + 1, chain_rows(MODE, K));
    if (!gathered_ok(records, records_bytes, G, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    if (!target_shard || (uses_draft(MODE) && !draft_shard) || !draft_tokens || !uniforms ||
        !out_tokens || !out_accept_len || !out_status)
        return SPEC_EINVAL;
    if (!buf_ok(out_sums, sums_bytes, shard_sums_slot(B, a.V)) ||
        !buf_ok(workspace, workspace_bytes, shard_ws_bytes(B)))
        return SPEC_EWORKSPACE;
    gathered_records(a, dtype, records);
    a.T = target_shard;
    a.D = draft_shard;
    a.tok = draft_tokens;
    a.u = uniforms;
    a.alpha = alpha;
    a.tau = tau;
    a.top_k = top_k;
    a.vec_t = vec_ok(target_shard, dtype, a.V);
    a.vec_d = uses_draft(MODE) && vec_ok(draft_shard, dtype, a.V);
    a.out_tok = out_tokens;
    a.out_len = out_accept_len;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_status = out_status;
    a.sums = static_cast<ChunkSums*>(out_sums);
    a.dec = static_cast<Decision*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)B * (unsigned)((a.C2 + kSweepGroups - 1) / kSweepGroups)), block(kSweepThreads);
    if (dtype == SPEC_BF16) return shard_launch(k_sweep<uint16_t, MODE, true>, grid, block, a, st);
    return shard_launch(k_sweep<float, MODE, true>, grid, block, a, st);
}

template <int MODE>
spec_status shard_sample(const void* target_shard, const void* draft_shard, spec_dtype dtype,
                         const void* sums, size_t sums_bytes, const float* uniforms, int B, int K, int V, int G,
                         int shard, int32_t* out_tokens, float* out_target_logprob,
                         float* out_behavior_logprob, int32_t* out_sample_shard, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, shard, chain_rows(MODE, K))) return SPEC_EINVAL;
    Args a = shard_args(dtype, B, K, V, G, shard, K + 1, chain_rows(MODE, K));
    if (!gathered_ok(sums, sums_bytes, G, shard_sums_slot(B, a.V))) return SPEC_EWORKSPACE;
    if (!target_shard || (uses_draft(MODE) && !draft_shard) || !uniforms || !out_tokens) return SPEC_EINVAL;
    if (!buf_ok(workspace, workspace_bytes, shard_ws_bytes(B))) return SPEC_EWORKSPACE;
    a.T = target_shard;
    a.D = draft_shard;
    a.u = uniforms;
    a.vec_t = vec_ok(target_shard, dtype, a.V);
    a.vec_d = uses_draft(MODE) && vec_ok(draft_shard, dtype, a.V);
    a.sums = static_cast<ChunkSums*>(const_cast<void*>(sums));
    a.sums_slot = shard_sums_slot(B, a.V);
    a.dec = static_cast<Decision*>(workspace);
    a.out_tok = out_tokens;
    a.out_tlp = out_target_logprob;
    a.out_blp = out_behavior_logprob;
    a.out_owner = out_sample_shard;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(B), block(kSampleThreads);
    if (dtype == SPEC_BF16) return shard_launch(k_sample<uint16_t, MODE, true>, grid, block, a, st);
    return shard_launch(k_sample<float, MODE, true>, grid, block, a, st);
}

}  // namespace

extern "C" {

spec_status spec_shard_sweep_exact(const void* target_shard, const void* draft_shard,
                                   spec_dtype dtype, const void* records, size_t records_bytes,
                                   const int32_t* draft_tokens, const float* uniforms, int B,
                                   int K, int V, int G, int shard, int32_t* out_tokens,
                                   int32_t* out_accept_len, float* out_target_logprob,
                                   float* out_behavior_logprob, int32_t* out_status,
                                   void* out_sums, size_t sums_bytes, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return shard_sweep<kExact>(target_shard, draft_shard, dtype, records, records_bytes, draft_tokens, uniforms, B, K, V, G,
                               shard, 0.f, 0.f, 0, out_tokens, out_accept_len, out_target_logprob,
                               out_behavior_logprob, out_status, out_sums, sums_bytes, workspace,
                               workspace_bytes, stream);
}

spec_status spec_shard_sweep_power(const void* target_shard, const void* draft_shard,
                                   spec_dtype dtype, const void* records, size_t records_bytes,
                                   const int32_t* draft_tokens, const float* uniforms, int B,
                                   int K, int V, int G, int shard, float alpha, int32_t* out_tokens,
                                   int32_t* out_accept_len, float* out_target_logprob,
                                   float* out_behavior_logprob, int32_t* out_status,
                                   void* out_sums, size_t sums_bytes, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return shard_sweep<kPower>(target_shard, draft_shard, dtype, records, records_bytes, draft_tokens, uniforms, B, K, V, G,
                               shard, alpha, 0.f, 0, out_tokens, out_accept_len, out_target_logprob,
                               out_behavior_logprob, out_status, out_sums, sums_bytes, workspace,
                               workspace_bytes, stream);
}

spec_status spec_shard_sample_exact(const void* target_shard, const void* draft_shard,
                                    spec_dtype dtype, const void* sums, size_t sums_bytes,
                                    const float* uniforms,
                                    int B, int K, int V, int G, int shard, int32_t* out_tokens,
                                    float* out_target_logprob, float* out_behavior_logprob,
                                    int32_t* out_sample_shard, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return shard_sample<kExact>(target_shard, draft_shard, dtype, sums, sums_bytes, uniforms, B, K, V, G, shard,
                                out_tokens, out_target_logprob, out_behavior_logprob, out_sample_shard,
                                workspace, workspace_bytes, stream);
}

spec_status spec_shard_sample_power(const void* target_shard, const void* draft_shard,
                                    spec_dtype dtype, const void* sums, size_t sums_bytes,
                                    const float* uniforms,
                                    int B, int K, int V, int G, int shard, int32_t* out_tokens,
                                    float* out_target_logprob, float* out_behavior_logprob,
                                    int32_t* out_sample_shard, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return shard_sample<kPower>(target_shard, draft_shard, dtype, sums, sums_bytes, uniforms, B, K, V, G, shard,
                                out_tokens, out_target_logprob, out_behavior_logprob, out_sample_shard,
                                workspace, workspace_bytes, stream);
}

size_t spec_shard_values_bytes(int B, int K) {
    if (B < 1 || B > kMaxB || K < 1 || K > SPEC_MAX_K) return 0;
    return align_up((size_t)B * K * sizeof(float), 256);
}

spec_status spec_shard_values_relaxed(const void* target_shard, spec_dtype dtype,
                                      const int32_t* draft_tokens, int B, int K, int V, int G,
                                      int shard, void* out_values, size_t values_bytes,
                                      void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, shard, K + 1)) return SPEC_EINVAL;
    if (!target_shard || !draft_tokens) return SPEC_EINVAL;
    if (!buf_ok(out_values, values_bytes, spec_shard_values_bytes(B, K))) return SPEC_EWORKSPACE;
    Args a = shard_args(dtype, B, K, V, G, shard, K + 1, K + 1);
    a.T = target_shard;
    a.tok = draft_tokens;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)((B * K + kThreads - 1) / kThreads)), block(kThreads);
    float* out = static_cast<float*>(out_values);
    if (dtype == SPEC_BF16)
        hipLaunchKernelGGL((k_values<uint16_t>), grid, block, 0, st, a, out);
    else
        hipLaunchKernelGGL((k_values<float>), grid, block, 0, st, a, out);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_shard_stats_relaxed(const void* target_shard, spec_dtype dtype,
                                     const int32_t* draft_tokens, const void* values,
                                     size_t values_bytes, int B, int K,
                                     int V, int G, int shard, void* out_record, size_t record_bytes,
                                     void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !shard_ok(dtype, B, K, V, G, shard, K + 1)) return SPEC_EINVAL;
    if (!gathered_ok(values, values_bytes, G, spec_shard_values_bytes(B, K))) return SPEC_EWORKSPACE;
    if (!target_shard || !draft_tokens) return SPEC_EINVAL;
    Args a = shard_args(dtype, B, K, V, G, shard, K + 1, K + 1);
    if (!buf_ok(out_record, record_bytes, shard_layout(dtype, B, a.R, a.V).slot)) return SPEC_EWORKSPACE;
    a.T = target_shard;
    a.tok = draft_tokens;
    a.vec_t = vec_ok(target_shard, dtype, a.V);
    a.xv_in = static_cast<const float*>(values);
    a.slot_xv = spec_shard_values_bytes(B, K) / sizeof(float);
    return shard_stats<kRelaxed, true>(a, dtype, out_record, static_cast<hipStream_t>(stream));
}

spec_status spec_shard_sweep_relaxed(const void* target_shard, spec_dtype dtype, const void* records,
                                     size_t records_bytes, const int32_t* draft_tokens, const float* uniforms, int B,
                                     int K, int V, int G, int shard, float tau, int top_k,
                                     int32_t* out_tokens, int32_t* out_accept_len,
                                     float* out_target_logprob, float* out_behavior_logprob,
                                     int32_t* out_status, void* out_sums, size_t sums_bytes,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return shard_sweep<kRelaxed>(target_shard, nullptr, dtype, records, records_bytes, draft_tokens, uniforms, B, K, V, G,
                                 shard, 0.f, tau, top_k, out_tokens, out_accept_len, out_target_logprob,
                                 out_behavior_logprob, out_status, out_sums, sums_bytes, workspace,
                                 workspace_bytes, stream);
}

spec_status spec_shard_sample_relaxed(const void* target_shard, spec_dtype dtype, const void* sums,
                                      size_t sums_bytes, const float* uniforms, int B, int K, int V, int G, int shard,
                                      int32_t* out_tokens, float* out_target_logprob,
                                      float* out_behavior_logprob, int32_t* out_sample_shard,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    return shard_sample<kRelaxed>(target_shard, nullptr, dtype, sums, sums_bytes, uniforms, B, K, V, G, shard,
                                  out_tokens, out_target_logprob, out_behavior_logprob, out_sample_shard,
                                  workspace, workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------- allocation-free call
// The exact rule's workspace in a file-scope device array, for callers that
// cannot allocate.  In host code `scratch` names a host-side stand-in, not
// the array: its device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on device d, once looked up

// The current device's address of the scratch array.
spec_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SPEC_OK;
}

// Zeroes n bytes (a multiple of 16) at p with vector stores: the single-launch
// protocol reads a zero word as "not published yet", and a call that timed out
// may have left words behind.  A kernel rather than hipMemsetAsync, so that the
// call can be captured into a HIP graph.
__global__ __launch_bounds__(kThreads) void k_zero(uint4* p, size_t n16) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * kThreads)
        p[i] = z;
}

}  // namespace

extern "C" spec_status spec_verify_exact_noalloc(const void* target_logits, const void* draft_logits,
                                                 spec_dtype dtype, const int32_t* draft_tokens,
                                                 const float* uniforms, int B, int K, int V,
                                                 int32_t* out_tokens, int32_t* out_accept_len,
                                                 float* out_target_logprob,
                                                 float* out_behavior_logprob, int32_t* out_status,
                                                 void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(dtype, B, K, V, 2 * K + 1)) return SPEC_EINVAL;
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !out_tokens ||
        !out_accept_len || !out_status)
        return SPEC_EINVAL;
    // the exact call's workspace layout at this dtype, as spec_verify_exact checks it
    const size_t need = make_layout(B, 2 * K + 1, tpr_of(dtype, V), c2_of(dtype, V)).total;
    if (need > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ESCRATCH;
    void* ws = nullptr;
    const spec_status s = scratch_on_current_device(&ws);
    if (s != SPEC_OK) return s;
    // need is a multiple of 256 (make_layout aligns every region)
    const size_t n16 = need / 16;
    if (n16 > 0) {
        const size_t want = (n16 + kThreads - 1) / kThreads;
        const unsigned blocks = (unsigned)(want < 1024 ? want : 1024);
        hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (uint4*)ws, n16);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    }
    return spec_verify_exact(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V,
                             out_tokens, out_accept_len, out_target_logprob, out_behavior_logprob,
                             out_status, ws, SPEC_NOALLOC_SCRATCH_BYTES, stream);
}
