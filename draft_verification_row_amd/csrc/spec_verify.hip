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
// How it is computed here (no kernel design comes from the pages):
//
//   pass 1  one workgroup per (request, row, vocabulary chunk).  Each thread
//           streams kP1Vecs 16-byte vectors of its chunk, widens bf16 to
//           fp32 exactly and keeps the row statistics the rule needs:
//           max and lowest-index argmax, sum exp(l - m) (v_exp_f32, fp32
//           per vector, fp64 across vectors), and the rank count
//           #{t : l_t > l_x}.  Waves reduce with cross-lane shuffles, the
//           four waves combine through LDS in a fixed order, and the chunk
//           partial is published to the workspace.  An atomic ticket per
//           request elects the last workgroup of the request, which gathers
//           the chunk partials of every row and combines them (fixed order,
//           fp64), evaluates the
//           acceptance tests of all K drafts at once (one lane per draft,
//           fp64), finds the first rejection with a wave ballot, and writes
//           the accepted prefix.  Greedy and tree calls finish here.
//
//   pass 2  (exact and relaxed) one workgroup per (request, chunk) sweeps
//           the row(s) the terminal token is drawn from, in fp64 with an
//           explicit Cody-Waite exp: exact normalizers sum_t exp(l_t - M)
//           for the target (and draft) row and, for a residual, the chunk
//           sums of exp(l - M) and exp(d - M_q) over the tokens with p > q.
//           The last workgroup of the request turns these into chunk masses
//           of relu(p - q) (or of p), picks the chunk holding u_K * Z by a
//           sequential prefix, rescans that one chunk with a block
//           exclusive scan and writes the token and its log-probs.
//
// Every reduction runs in a fixed order, so results are bitwise
// reproducible.  No float atomics are used; atomics only elect the last
// workgroup.
//
// Cross-workgroup hand-off.  The workgroups of one request run on all eight
// XCDs, whose L2 caches are not coherent with each other.  A release/acquire
// fence at device scope would make every workgroup write back and invalidate
// its whole L2, which stalls the streaming kernel.  Instead each partial is
// published as 64-bit words that carry a tag in their upper half
// (payload | kTag << 32), written and read with relaxed device-scope atomics,
// which the hardware keeps coherent across XCDs without cache maintenance.
// Each word validates itself, so no ordering between words is needed: the
// elected workgroup reads every word, re-reads (with a bounded wait) any
// whose tag has not arrived yet, and writes zeros back, so the workspace is
// all zeros between calls.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileVecs = 2;  // 16-byte vectors per thread per streaming tile
constexpr int kWgPerCu = 8;   // streaming workgroups per compute unit
constexpr int kMaxGrid = 8192;
constexpr int kP2Vecs = 2;  // 16-byte vectors per thread per pass-2 chunk
constexpr int kMaxRows = 2 * SPEC_MAX_K + 1;
constexpr int kMaxB = SPEC_MAX_B;
// Per-request tickets of pass 2, one 128-byte line each: atomics on a line
// shared by several requests serialize behind each other.  Zero at rest.
constexpr int kCtrlStride = 32;  // int32 per request
constexpr size_t kCtrlBytes = (size_t)kMaxB * kCtrlStride * 4;
constexpr int kMaxC2 = 256;  // pass-2 chunks per row at SPEC_MAX_V (bf16 and fp32)
static_assert(SPEC_MAX_V <= kMaxC2 * kThreads * kP2Vecs * 4, "pass-2 chunk table too small");
static_assert(kMaxC2 <= kThreads, "one pass-2 chunk per thread in the terminal scan");
constexpr uint32_t kTag = 0x5ec0fa11u;
constexpr int kMaxSpins = 1 << 20;  // bounded wait for a published word (~60 ms)

enum Mode { kGreedy = 0, kExact = 1, kRelaxed = 2, kTree = 3 };

// Statistics of one row segment, written by the streaming kernel and read by
// the next kernel on the stream (the launch boundary makes them visible):
// max, lowest index of the max, rank count, sum exp(l - max).
struct alignas(8) Seg {
    float m;
    int idx;
    int cnt;
    int pad;
    double s;
};

// Chunk partial of pass 2 (eight tagged words = four fp64 sums): sum of
// a = exp(l - Mt) and b = exp(d - Md) over the chunk, and over its tokens
// with p > q.
constexpr int kP2Words = 8;

struct Layout {
    size_t seg, p2, total;
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline Layout make_layout(int B, int R, int C2) {
    Layout L;
    // one segment record per (streaming workgroup, row it touches): ids w + row
    L.seg = kCtrlBytes;
    L.p2 = align_up(L.seg + ((size_t)kMaxGrid + (size_t)B * R) * sizeof(Seg), 256);
    L.total = align_up(L.p2 + (size_t)B * C2 * kP2Words * 8, 256);
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

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bit patterns
    static constexpr int kVec = 8;
    __device__ static inline float at(const uint16_t* p, size_t i) {
        return __uint_as_float((uint32_t)p[i] << 16);
    }
    template <int AUX = 0>
    __device__ static inline u32x4 vraw(__amdgpu_buffer_rsrc_t r, int e) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, e * 2, 0, AUX);
    }
    __device__ static inline float sraw(__amdgpu_buffer_rsrc_t r, int e) {
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, e * 2, 0, 0) << 16);
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
};

template <>
struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static inline float at(const float* p, size_t i) { return p[i]; }
    template <int AUX = 0>
    __device__ static inline u32x4 vraw(__amdgpu_buffer_rsrc_t r, int e) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, AUX);
    }
    __device__ static inline float sraw(__amdgpu_buffer_rsrc_t r, int e) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, e * 4, 0, 0));
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
};

// Loads this thread's NV vectors of the chunk [c0, c1): vector k holds
// elements c0 + (k * kThreads + tid) * VEC + [0, VEC).  Elements at or past
// c1 read as -inf.  `vec` selects the 16-byte path (row start and size
// 16-byte aligned); otherwise each element is loaded on its own.  AUX is the
// cache-policy field of the vector loads (kStream: read once, do not keep).
constexpr int kStream = 2;
template <typename T, int NV, int AUX = 0>
__device__ inline void load_chunk(__amdgpu_buffer_rsrc_t r, int c0, int c1, bool vec,
                                  float (&v)[NV][Elem<T>::kVec]) {
    constexpr int VEC = Elem<T>::kVec;
    const int t0 = c0 + (int)threadIdx.x * VEC;
    if (vec) {
        u32x4 q[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) q[k] = Elem<T>::template vraw<AUX>(r, t0 + k * kThreads * VEC);
#pragma unroll
        for (int k = 0; k < NV; ++k) Elem<T>::unpack(q[k], v[k]);
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int i = 0; i < VEC; ++i) v[k][i] = Elem<T>::sraw(r, t0 + k * kThreads * VEC + i);
    }
    if (c1 - c0 < NV * kThreads * VEC) {  // partial chunk (uniform per workgroup)
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                if (t0 + k * kThreads * VEC + i >= c1) v[k][i] = -INFINITY;
    }
}

// Loads NV vectors of consecutive tokens [e0, e0 + NV*VEC) (one thread's
// contiguous run); tokens at or past V read as -inf.
template <typename T, int NV>
__device__ inline void load_run(__amdgpu_buffer_rsrc_t r, int e0, int V, bool vec,
                                float (&v)[NV * Elem<T>::kVec]) {
    constexpr int VEC = Elem<T>::kVec;
    if (vec) {
        u32x4 q[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) q[k] = Elem<T>::vraw(r, e0 + k * VEC);
#pragma unroll
        for (int k = 0; k < NV; ++k) Elem<T>::unpack(q[k], v + k * VEC);
    } else {
#pragma unroll
        for (int i = 0; i < NV * VEC; ++i) v[i] = Elem<T>::sraw(r, e0 + i);
    }
#pragma unroll
    for (int i = 0; i < NV * VEC; ++i)
        if (e0 + i >= V) v[i] = -INFINITY;
}

// ------------------------------------------------------------ fp64 exp(x<=0)
// Cody-Waite reduction x = k ln2/64 + r, |r| <= ln2/128, then a degree-4
// Taylor polynomial (truncation error r^5/120 < 4e-14 relative) and
// 2^(k/64) = 2^(k>>6) * tab[k & 63].  Branch-free and built from full-rate
// fp64 fma/add/mul and integer ops only: adding 1.5*2^52 leaves round(y) in
// the low word of the double, and 2^(k>>6) is applied by adding (k>>6) to the
// exponent field of tab[k & 63] (results stay normal for x > -700).  x <= -700
// (and -inf) gives exactly 0.
constexpr double kInvLn2x64 = 92.332482616893656877;   // 64 / ln 2
constexpr double kLn2o64Hi = 0.010830424726009368896;  // ln2/64 rounded to 24 bits
constexpr double kLn2o64Lo = -2.9760223436840126e-11;  // ln2/64 - hi
constexpr double kRoundMagic = 6755399441055744.0;     // 1.5 * 2^52

__device__ inline double exp_nonpos(double x, const double* tab) {
    const double xc = fmax(x, -700.0);
    const double t = fma(xc, kInvLn2x64, kRoundMagic);
    const int k = (int)(uint32_t)__double_as_longlong(t);  // round(xc * 64/ln2)
    const double kd = t - kRoundMagic;
    double r = fma(-kd, kLn2o64Hi, xc);
    r = fma(-kd, kLn2o64Lo, r);
    double p = fma(r, 1.0 / 24.0, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    const long long tb = __double_as_longlong(tab[k & 63]) + ((long long)(k >> 6) << 52);
    const double e = __longlong_as_double(tb) * p;
    return (x > -700.0) ? e : 0.0;
}

__device__ inline void fill_exp_table(double* tab) {
    if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
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

// ------------------------------------------------- tagged-word hand-off
__device__ inline void put_word(uint64_t* p, uint32_t v) {
    __hip_atomic_store(p, ((uint64_t)kTag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void put_double(uint64_t* p, double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    put_word(p, (uint32_t)u);
    put_word(p + 1, (uint32_t)(u >> 32));
}

// Reads n tagged words into out[], waiting (bounded) for any not yet
// published, then returns them to zero.  Returns false on timeout.
template <int N>
__device__ inline bool take_words(uint64_t* p, uint32_t* out) {
    uint64_t w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int spins = 0;
        while ((uint32_t)(w[i] >> 32) != kTag) {
            if (++spins > kMaxSpins) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            w[i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        out[i] = (uint32_t)w[i];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) __hip_atomic_store(p + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return ok;
}

__device__ inline double join_double(uint32_t lo, uint32_t hi) {
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ inline int ticket_add(int* t) {
    return __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void ticket_reset(int* t) {
    __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    int G;       // streaming workgroups
    int C2;      // pass-2 chunks per row
    int vec_t, vec_d;
    float tau;
    int top_k;
    int32_t* out_tok;
    int32_t* out_len;
    float* out_tlp;
    float* out_blp;
    int32_t* out_status;
    int32_t* out_path;
    int L;  // output row length: K+1, or N for a tree
    unsigned char* ws;
};

__device__ inline int* ticket2(const Args& a, int b) {
    return reinterpret_cast<int*>(a.ws) + kCtrlStride * b;
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The streaming split: all tiles of the call (row-major: global row g of the
// call, then tile c of the row) are cut into G contiguous, equal ranges.
__host__ __device__ inline int split_lo(long long total, int G, int w) { return (int)(total * w / G); }
// workgroup whose range holds tile t
__host__ __device__ inline int split_owner(long long total, int G, long long t) {
    return (int)(((t + 1) * G - 1) / total);
}

template <typename T>
__device__ inline const T* uniform_ptr(const T* p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = (uint32_t)uniform((int)(uint32_t)u), hi = (uint32_t)uniform((int)(uint32_t)(u >> 32));
    return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Logit row g of the call (request g / R, row g % R of that request).  The
// result is wave-uniform, so loads use a scalar base and 32-bit offsets.
template <typename T, int MODE>
__device__ inline const T* call_row(const Args& a, int g, int& vec, int& active) {
    const int b = g / a.R, rr = g - (g / a.R) * a.R;
    active = 1;
    if (MODE == kTree && a.num_nodes) active = uniform(rr < min(max(a.num_nodes[b], 1), a.rows_t));
    if (MODE == kExact && rr >= a.rows_t) {
        vec = a.vec_d;
        return uniform_ptr(reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + (rr - a.rows_t)) * a.V);
    }
    vec = a.vec_t;
    return uniform_ptr(reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + rr) * a.V);
}

// Issues this thread's loads of tile c of a row: vector k covers tokens
// c*TILE + (k*kThreads + tid)*VEC + [0, VEC).  Indices are clamped into the
// row and the caller masks tokens past V, so no load leaves the row.
template <typename T, bool NT, bool VECP>
__device__ inline void load_tile(const T* row, int V, int c, u32x4 (&q)[kTileVecs]) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int TILE = kThreads * kTileVecs * VEC;
    const int t0 = c * TILE + (int)threadIdx.x * VEC;
    if (VECP) {  // V is a multiple of VEC and every row is 16-byte aligned
#pragma unroll
        for (int k = 0; k < kTileVecs; ++k) {
            // global address space: global loads wait on vmcnt only, so the
            // look-ahead loads stay in flight while this tile is reduced
            const gu32x4* p = (const gu32x4*)(row + min(t0 + k * kThreads * VEC, V - VEC));
            q[k] = NT ? __builtin_nontemporal_load(p) : *p;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kTileVecs; ++k) q[k] = Elem<T>::gather_clamped(row, t0 + k * kThreads * VEC, V);
    }
}

// ----------------------------------------------------------- streaming pass
// Every logit row is read once.  Workgroup w walks tiles [lo(w), lo(w+1))
// with one tile of look-ahead and keeps per-thread running statistics; at
// the end of each row segment it reduces them over the workgroup and writes
// one Seg record, id w + row.  Per element: widen, max (and argmax), and for
// the normalizer one fma, one exp2 and one add.
// VECP: every row of the call takes the 16-byte path (chosen on the host).
template <typename T, int MODE, bool SUM, bool VECP>
__global__ __launch_bounds__(kThreads, kWgPerCu) void k_stream(const Args a) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int TILE = kThreads * kTileVecs * VEC;
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    constexpr bool COUNT = (MODE == kRelaxed);
    constexpr bool NT = ARGMAX;  // greedy and tree never revisit a row

    Seg* segs = reinterpret_cast<Seg*>(a.ws + make_layout(a.B, a.R, a.C2).seg);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    __shared__ double tab[64];
    __shared__ float s_m[kWaves];
    __shared__ int s_i[kWaves];
    __shared__ int s_c[kWaves];
    __shared__ double s_s[kWaves];
    if (SUM) fill_exp_table(tab);
    __syncthreads();

    const long long total = (long long)a.B * a.R * a.tpr;
    const int w = blockIdx.x;
    const int t_lo = split_lo(total, gridDim.x, w), t_hi = split_lo(total, gridDim.x, w + 1);
    if (t_lo >= t_hi) return;
    int g = uniform(t_lo / a.tpr);
    int c = uniform(t_lo - g * a.tpr);
    int vec, act, nvec, nact;
    const T* row = call_row<T, MODE>(a, g, vec, act);
    const T* nrow = row;
    u32x4 qn[kTileVecs];
    if (act) load_tile<T, NT, VECP>(row, a.V, c, qn);

    auto rank_threshold = [&](int gg, const T* rp) -> float {
        const int b = gg / a.R, rr = gg - (gg / a.R) * a.R;
        if (!COUNT || rr >= a.K) return INFINITY;
        const int x = a.tok[b * a.K + rr];
        return ((unsigned)x < (unsigned)a.V) ? Elem<T>::at(rp, (size_t)x) : INFINITY;
    };
    float thr = COUNT ? rank_threshold(g, row) : INFINITY;

    float m = -INFINITY, mL = -INFINITY;
    int idx = INT_MAX, cnt = 0;
    double s = 0.0;
    for (int t = t_lo; t < t_hi; ++t) {
        u32x4 q[kTileVecs];
#pragma unroll
        for (int k = 0; k < kTileVecs; ++k) q[k] = qn[k];
        const bool row_end = (c + 1 == a.tpr);
        nvec = vec;
        nact = act;
        if (t + 1 < t_hi) {  // look ahead one tile
            if (row_end) {
                nrow = call_row<T, MODE>(a, g + 1, nvec, nact);
                if (nact) load_tile<T, NT, VECP>(nrow, a.V, 0, qn);
            } else if (act) {
                load_tile<T, NT, VECP>(row, a.V, c + 1, qn);
            }
        }
        if (act) {
            const int t0 = c * TILE + (int)threadIdx.x * VEC;
            float v[kTileVecs][VEC];
#pragma unroll
            for (int k = 0; k < kTileVecs; ++k) Elem<T>::unpack(q[k], v[k]);
            if (row_end && a.V % TILE != 0) {  // ragged last tile: clamped lanes
#pragma unroll
                for (int k = 0; k < kTileVecs; ++k)
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        if (t0 + k * kThreads * VEC + i >= a.V) v[k][i] = -INFINITY;
            }
            float tm = -INFINITY;
#pragma unroll
            for (int k = 0; k < kTileVecs; ++k) {
                const int base = t0 + k * kThreads * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    if (ARGMAX) {
                        if (v[k][i] > m) {
                            m = v[k][i];
                            idx = base + i;
                        }
                    } else {
                        tm = fmaxf(tm, v[k][i]);
                    }
                    if (COUNT) cnt += (v[k][i] > thr) ? 1 : 0;
                }
            }
            if (!ARGMAX) m = fmaxf(m, tm);
            if (SUM && m > -INFINITY) {
                // Running sum of 2^(l*L - mL) against a reference mL = fl(m*L)
                // that only moves up (the sum is rescaled when it does).
                const float nL = m * kLog2e;
                if (nL > mL) {
                    s *= (double)__builtin_amdgcn_exp2f(mL - nL);
                    mL = nL;
                }
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < kTileVecs; ++k)
#pragma unroll
                    for (int i = 0; i < VEC; ++i) acc += __builtin_amdgcn_exp2f(fmaf(v[k][i], kLog2e, -mL));
                s += (double)acc;
            }
        }
        if (row_end || t + 1 == t_hi) {
            // ---- end of a row segment: reduce over the workgroup, write it
            if (act) {
                float M = m;
                int I = idx;
                if (ARGMAX)
                    wave_argmax(M, I);
                else
                    M = wave_max(M);
                if (lane == 0) {
                    s_m[wave] = M;
                    s_i[wave] = I;
                }
                __syncthreads();
                M = s_m[0];
                I = s_i[0];
#pragma unroll
                for (int ww = 1; ww < kWaves; ++ww) argmax_combine(M, I, s_m[ww], s_i[ww]);
                double st = 0.0;
                if (SUM && M > -INFINITY && m > -INFINITY)  // times 2^(mL - M*L), in fp64
                    st = s * exp_nonpos(((double)mL - (double)M * (double)kLog2e) * kLn2, tab);
                if (SUM) st = wave_sum(st);
                const int ct = COUNT ? wave_sum_i(cnt) : 0;
                if (lane == 0) {
                    s_s[wave] = st;
                    s_c[wave] = ct;
                }
                __syncthreads();
                if (threadIdx.x == 0) {
                    Seg sg;
                    sg.m = M;
                    sg.idx = I;
                    sg.cnt = 0;
                    sg.pad = 0;
                    sg.s = 0.0;
#pragma unroll
                    for (int ww = 0; ww < kWaves; ++ww) {
                        sg.s += s_s[ww];
                        sg.cnt += s_c[ww];
                    }
                    segs[(size_t)w + g] = sg;
                }
                __syncthreads();  // s_* are reused by the next segment
            }
            m = -INFINITY;
            mL = -INFINITY;
            idx = INT_MAX;
            cnt = 0;
            s = 0.0;
        }
        if (row_end) {
            ++g;
            c = 0;
            row = nrow;
            vec = nvec;
            act = nact;
            if (COUNT && t + 1 < t_hi) thr = rank_threshold(g, row);
        } else {
            ++c;
        }
    }
}

// ------------------------------------------------------- row statistics
// Combines the Seg records of rows [0, rows) of request b into row max M,
// argmax g (lowest index), rank count c and log normalizer lnS, in LDS.
// Segments are gathered one per thread (kThreads per batch); each row then
// folds its segments in ascending order.  Deterministic.
struct RowStats {
    float M[kMaxRows];
    int g[kMaxRows];
    int c[kMaxRows];
    double lnS[kMaxRows];
    // scratch
    double S[kMaxRows];
    float bM[kMaxRows];
    int off[kMaxRows + 1];
    int w0[kMaxRows];
    float qm[kThreads];
    int qi[kThreads];
    int qc[kThreads];
    double qs[kThreads];
};

template <bool SUM>
__device__ void gather_rows(const Args& a, int b, int rows, RowStats& rs) {
    const Seg* segs = reinterpret_cast<const Seg*>(a.ws + make_layout(a.B, a.R, a.C2).seg);
    const long long total = (long long)a.B * a.R * a.tpr;
    for (int r = threadIdx.x; r < rows; r += kThreads) {
        const long long rg = (long long)b * a.R + r;
        const int w0 = split_owner(total, a.G, rg * a.tpr), w1 = split_owner(total, a.G, (rg + 1) * a.tpr - 1);
        rs.w0[r] = w0;
        rs.off[r + 1] = w1 - w0 + 1;
        rs.M[r] = -INFINITY;
        rs.g[r] = INT_MAX;
        rs.c[r] = 0;
        rs.S[r] = 0.0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        rs.off[0] = 0;
        for (int r = 0; r < rows; ++r) rs.off[r + 1] += rs.off[r];
    }
    __syncthreads();
    const int nslots = rs.off[rows];
    for (int base = 0; base < nslots; base += kThreads) {
        const int si = base + (int)threadIdx.x;
        int sr = 0;
        if (si < nslots) {
            while (rs.off[sr + 1] <= si) ++sr;
            const Seg sg = segs[(size_t)rs.w0[sr] + (si - rs.off[sr]) + (size_t)b * a.R + sr];
            rs.qm[threadIdx.x] = sg.m;
            rs.qi[threadIdx.x] = sg.idx;
            rs.qc[threadIdx.x] = sg.cnt;
            rs.qs[threadIdx.x] = sg.s;
        }
        __syncthreads();
        const int bend = min(base + kThreads, nslots);
        for (int r = threadIdx.x; r < rows; r += kThreads) {
            const int lo = max(base, rs.off[r]), hi = min(bend, rs.off[r + 1]);
            if (lo >= hi) continue;
            float M = -INFINITY;
            int g = INT_MAX, C = 0;
            for (int q = lo; q < hi; ++q) {
                argmax_combine(M, g, rs.qm[q - base], rs.qi[q - base]);
                C += rs.qc[q - base];
            }
            rs.bM[r] = M;
            float RM = rs.M[r];
            int RG = rs.g[r];
            argmax_combine(RM, RG, M, g);
            rs.g[r] = RG;
            rs.c[r] += C;
            if (!SUM) rs.M[r] = RM;
        }
        __syncthreads();
        if (SUM) {
            if (si < bend) {  // rescale this segment's sum to its batch row max
                const float mq = rs.qm[threadIdx.x];
                rs.qs[threadIdx.x] = (mq > -INFINITY) ? rs.qs[threadIdx.x] * exp((double)mq - (double)rs.bM[sr]) : 0.0;
            }
            __syncthreads();
            for (int r = threadIdx.x; r < rows; r += kThreads) {
                const int lo = max(base, rs.off[r]), hi = min(bend, rs.off[r + 1]);
                if (lo >= hi) continue;
                double S = 0.0;
                for (int q = lo; q < hi; ++q) S += rs.qs[q - base];
                const float M = rs.bM[r], RM = rs.M[r];
                if (M > RM) {
                    rs.S[r] = (RM > -INFINITY ? rs.S[r] * exp((double)RM - (double)M) : 0.0) + S;
                    rs.M[r] = M;
                } else if (M > -INFINITY) {
                    rs.S[r] += S * exp((double)M - (double)RM);
                }
            }
            __syncthreads();
        }
    }
    for (int r = threadIdx.x; r < rows; r += kThreads) rs.lnS[r] = log(rs.S[r]);
    __syncthreads();
}

// ------------------------------------------------------ chain decision
// Lane j < K of wave 0 evaluates the test of draft j; a ballot finds the
// first rejection n (lane K never accepts, so n <= K).  Results go to LDS.
struct ChainDecision {
    int n, bad_n;
    int x[64];
    double lp[64], lq[64], lx[64], dx[64];
};

template <typename T, int MODE>
__device__ void chain_decide(const Args& a, int b, const RowStats& rs, ChainDecision& cd) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        const int j = lane, K = a.K;
        bool acc = false, bad = false;
        int x = -1;
        double lp = 0.0, lq = 0.0, lx = -INFINITY, dx = -INFINITY;
        if (j < K) {
            x = a.tok[b * K + j];
            bad = (unsigned)x >= (unsigned)a.V;
            if (!bad) {
                if (MODE == kGreedy) {
                    acc = (x == rs.g[j]);
                    lp = -rs.lnS[j];  // the accepted token is the row max
                } else {
                    const T* Tp = reinterpret_cast<const T*>(a.T);
                    lx = Elem<T>::at(Tp, (size_t)(b * a.rows_t + j) * a.V + x);
                    lp = (lx - (double)rs.M[j]) - rs.lnS[j];
                    if (MODE == kExact) {
                        const T* Dp = reinterpret_cast<const T*>(a.D);
                        dx = Elem<T>::at(Dp, (size_t)(b * K + j) * a.V + x);
                        lq = (dx - (double)rs.M[a.rows_t + j]) - rs.lnS[a.rows_t + j];
                        double r;
                        if (lp == -INFINITY)
                            r = 0.0;
                        else if (lq == -INFINITY)
                            r = INFINITY;
                        else
                            r = exp(lp - lq);
                        acc = (double)a.u[b * (K + 1) + j] < r;
                    } else {
                        acc = (rs.c[j] < a.top_k) || (exp(lp) >= (double)a.tau);
                    }
                }
            }
        }
        const unsigned long long mask = __ballot(acc);
        const int n = __builtin_ctzll(~mask);
        cd.x[j] = x;
        cd.lp[j] = lp;
        cd.lq[j] = lq;
        cd.lx[j] = lx;
        cd.dx[j] = dx;
        if (j == n) {
            cd.n = n;
            cd.bad_n = (n < K && bad) ? 1 : 0;
        }
    }
    __syncthreads();
}

// Writes positions j < n (accepted drafts) and n < j < L (padding) of the
// chain outputs, plus accept_len and status.  Position n is the caller's.
template <int MODE>
__device__ void write_prefix(const Args& a, int b, const ChainDecision& cd) {
    const int n = cd.n, L = a.L;
    int32_t* otok = a.out_tok + (size_t)b * L;
    float* otlp = a.out_tlp ? a.out_tlp + (size_t)b * L : nullptr;
    float* oblp = a.out_blp ? a.out_blp + (size_t)b * L : nullptr;
    for (int j = threadIdx.x; j < L; j += kThreads) {
        if (j < n) {
            otok[j] = cd.x[j];
            if (otlp) otlp[j] = (float)cd.lp[j];
            if (oblp) oblp[j] = (MODE == kExact) ? (float)fmin(0.0, cd.lp[j] - cd.lq[j]) : 0.f;
        } else if (j > n) {
            otok[j] = -1;
            if (otlp) otlp[j] = 0.f;
            if (oblp) oblp[j] = 0.f;
        }
    }
    if (threadIdx.x == 0) {
        a.out_len[b] = n;
        a.out_status[b] = cd.bad_n;
    }
}

// -------------------------------------------------- greedy and tree: decide
template <typename T, int MODE, bool SUM>
__global__ __launch_bounds__(kThreads) void k_decide(const Args a) {
    const int b = blockIdx.x;
    __shared__ RowStats rs;
    const int nb = (MODE == kTree && a.num_nodes) ? min(max(a.num_nodes[b], 1), a.rows_t) : a.rows_t;
    gather_rows<SUM>(a, b, MODE == kTree ? nb : a.R, rs);
    if (MODE == kGreedy) {
        __shared__ ChainDecision cd;
        chain_decide<T, kGreedy>(a, b, rs, cd);
        write_prefix<kGreedy>(a, b, cd);
        if (threadIdx.x == 0) {
            const int n = cd.n;
            a.out_tok[(size_t)b * a.L + n] = rs.g[n];
            if (a.out_tlp) a.out_tlp[(size_t)b * a.L + n] = (float)(-rs.lnS[n]);
            if (a.out_blp) a.out_blp[(size_t)b * a.L + n] = 0.f;
        }
        return;
    }
    // tree: a node is accepted iff its token is its parent's argmax and its
    // parent is accepted; parents precede children
    __shared__ int t_par[SPEC_MAX_NODES];
    __shared__ int t_match[SPEC_MAX_NODES];
    __shared__ int t_path[SPEC_MAX_NODES];
    __shared__ int t_d, t_e, t_bad;
    const int N = a.rows_t;
    if (threadIdx.x < 64) {
        const int i = threadIdx.x;
        bool bad = false;
        if (i >= 1 && i < nb) {
            const int p = a.parents[b * N + i];
            const int t = a.tok[b * N + i];
            bad = !(p >= 0 && p < i && (unsigned)t < (unsigned)a.V);
            t_par[i] = bad ? -1 : p;
            t_match[i] = bad ? 0 : (t == rs.g[p]);
        }
        const unsigned long long bm = __ballot(bad);
        if (i == 0) t_bad = bm != 0ull;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long accm = 1ull;  // bit i: node i accepted
        int depth[SPEC_MAX_NODES];
        depth[0] = 0;
        int e = 0;
        for (int i = 1; i < nb; ++i) {
            const int p = t_par[i];
            depth[i] = 0;
            if (p >= 0 && t_match[i] && ((accm >> p) & 1ull)) {
                accm |= 1ull << i;
                depth[i] = depth[p] + 1;
                if (depth[i] > depth[e]) e = i;
            }
        }
        const int d = depth[e];
        for (int v = e, k = d - 1; k >= 0; --k, v = t_par[v]) t_path[k] = v;
        t_d = d;
        t_e = e;
    }
    __syncthreads();
    const int d = t_d, e = t_e;
    for (int k = threadIdx.x; k < N; k += kThreads) {
        int32_t* otok = a.out_tok + (size_t)b * N;
        if (k < d) {
            const int v = t_path[k];
            a.out_path[(size_t)b * N + k] = v;
            otok[k] = a.tok[b * N + v];
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

// -------------------------------------------------------------------- pass 2
// Block-wide sums and scans in a fixed order (deterministic).
__device__ inline double block_sum(double v, double* scratch) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kWaves; ++w) t += scratch[w];
    return t;
}

// Scan of v over threads in thread order.  Returns the inclusive prefix;
// *excl receives the previous thread's inclusive prefix (0 for thread 0), so
// the intervals [excl, incl) of consecutive threads tile [0, total) exactly.
__device__ inline double block_scan(double v, double* scratch, double* all, double* excl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += scratch[w];
    all[threadIdx.x] = v;
    __syncthreads();
    *excl = threadIdx.x ? all[threadIdx.x - 1] : 0.0;
    return v;
}

// Block-wide int max / min (every thread gets the result).
__device__ inline int block_max_i(int v, int* scratch) {
    v = wave_max_i(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = scratch[0];
    for (int w = 1; w < kWaves; ++w) r = max(r, scratch[w]);
    return r;
}

__device__ inline int block_min_i(int v, int* scratch) {
    v = wave_min_i(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = scratch[0];
    for (int w = 1; w < kWaves; ++w) r = min(r, scratch[w]);
    return r;
}

template <typename T, bool EXACT>
__global__ __launch_bounds__(kThreads) void k_pass2(const Args a) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int PER = kP2Vecs * VEC;  // tokens per thread
    constexpr int CH = kThreads * PER;
    uint64_t* slots = reinterpret_cast<uint64_t*>(a.ws + make_layout(a.B, a.R, a.C2).p2);

    const int b = blockIdx.x / a.C2;
    const int c = blockIdx.x % a.C2;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    __shared__ double tab[64];
    __shared__ double red[kWaves][4];
    __shared__ double scr[kWaves];
    __shared__ double scan_all[kThreads];
    __shared__ int iscr[kWaves];
    __shared__ int s_last;
    fill_exp_table(tab);

    // Every workgroup of the request derives the same decision from the
    // streamed row statistics (deterministic), then works on the row(s) the
    // terminal token is drawn from: target row n, and draft row n for a
    // residual.
    __shared__ RowStats rs;
    __shared__ ChainDecision cd;
    gather_rows<true>(a, b, a.R, rs);
    chain_decide<T, EXACT ? kExact : kRelaxed>(a, b, rs, cd);
    const int n = cd.n;
    const bool residual = EXACT && n < a.K;
    const T* trow = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + n) * a.V;
    const T* drow = residual ? reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + n) * a.V : trow;
    const double Mt = rs.M[n], Md = residual ? (double)rs.M[a.rows_t + n] : 0.0;
    // p > q  <=>  (l - Mt) - (d - Md) > lnSt - lnSd (streamed normalizers)
    const double cls = residual ? rs.lnS[n] - rs.lnS[a.rows_t + n] : 0.0;
    const __amdgpu_buffer_rsrc_t rt = row_rsrc(trow, a.V);
    const __amdgpu_buffer_rsrc_t rd = row_rsrc(drow, a.V);
    __syncthreads();

    // ---- sweep: fp64 sums over this chunk (coalesced, interleaved layout)
    {
        const int c0 = c * CH;
        const int c1 = min(c0 + CH, a.V);
        float vt[kP2Vecs][VEC], vd[kP2Vecs][VEC];
        // both rows are always loaded (rd aliases the target row when no
        // draft row is needed) so that all loads issue before any wait
        load_chunk<T, kP2Vecs>(rt, c0, c1, a.vec_t, vt);
        load_chunk<T, kP2Vecs>(rd, c0, c1, residual ? a.vec_d : a.vec_t, vd);
        double sa = 0.0, sb = 0.0, pa = 0.0, pb = 0.0;
#pragma unroll
        for (int k = 0; k < kP2Vecs; ++k)
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const double xa = (double)vt[k][i] - Mt;
                const double ea = exp_nonpos(xa, tab);
                sa += ea;
                if (residual) {
                    const double xb = (double)vd[k][i] - Md;
                    const double eb = exp_nonpos(xb, tab);
                    sb += eb;
                    if (xa - xb > cls) {
                        pa += ea;
                        pb += eb;
                    }
                }
            }
        sa = wave_sum(sa);
        if (residual) {
            sb = wave_sum(sb);
            pa = wave_sum(pa);
            pb = wave_sum(pb);
        }
        if (lane == 0) {
            red[wave][0] = sa;
            red[wave][1] = sb;
            red[wave][2] = pa;
            red[wave][3] = pb;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double t[4] = {0.0, 0.0, 0.0, 0.0};
            for (int w = 0; w < kWaves; ++w)
                for (int i = 0; i < 4; ++i) t[i] += red[w][i];
            uint64_t* w = slots + ((size_t)b * a.C2 + c) * kP2Words;
            for (int i = 0; i < 4; ++i) put_double(w + 2 * i, t[i]);
            s_last = (ticket_add(ticket2(a, b)) == a.C2 - 1);
        }
        __syncthreads();
        if (!s_last) return;
    }

    // ---- terminal sample (last workgroup of the request)
    // Chunk partials, one chunk per thread (a.C2 <= kThreads).
    __shared__ int s_bad_ws;
    __shared__ double s_base, s_Z;
    __shared__ int s_y, s_ylast, s_yany;
    if (threadIdx.x == 0) s_bad_ws = 0;
    __syncthreads();
    double csa = 0.0, csb = 0.0, cpa = 0.0, cpb = 0.0;
    if ((int)threadIdx.x < a.C2) {
        uint32_t w[kP2Words];
        if (!take_words<kP2Words>(slots + ((size_t)b * a.C2 + threadIdx.x) * kP2Words, w)) s_bad_ws = 1;
        csa = join_double(w[0], w[1]);
        csb = join_double(w[2], w[3]);
        cpa = join_double(w[4], w[5]);
        cpb = join_double(w[6], w[7]);
    }
    const double S = block_sum(csa, scr);
    const double Sq = residual ? block_sum(csb, scr) : 0.0;
    const double iS = 1.0 / S, iSq = residual ? 1.0 / Sq : 0.0;
    // residual mass of this chunk (clamped: tokens classified with the pass-1
    // normalizers can leave a rounding-size negative); fall back to p when
    // relu(p - q) has no mass
    double W = residual ? fmax(cpa * iS - cpb * iSq, 0.0) : csa;
    const double Zr = residual ? block_sum(W, scr) : 0.0;
    const bool res = residual && (Zr > 0.0);
    if (residual && !res) W = csa;
    const double Z = res ? Zr : S;
    const double target = (double)a.u[b * (a.K + 1) + a.K] * Z;
    double excl;
    const double incl = block_scan(W, scr, scan_all, &excl);
    // the unique chunk whose interval [excl, incl) holds target; if rounding
    // pushed target past the last boundary, the last chunk with mass
    const bool mine = (int)threadIdx.x < a.C2 && W > 0.0 && excl <= target && target < incl;
    int cstar = block_max_i(mine ? (int)threadIdx.x : -1, iscr);
    if (cstar < 0) cstar = block_max_i(((int)threadIdx.x < a.C2 && W > 0.0) ? (int)threadIdx.x : -1, iscr);
    cstar = max(cstar, 0);
    if ((int)threadIdx.x == cstar) s_base = excl;
    if (threadIdx.x == 0) s_Z = Z;
    __syncthreads();

    // ---- rescan chunk cstar; thread t owns tokens [e0 + t*PER, +PER)
    {
        const int e0 = cstar * CH + (int)threadIdx.x * PER;
        float lt_[PER], ld_[PER];
        load_run<T, kP2Vecs>(rt, e0, a.V, a.vec_t, lt_);
        load_run<T, kP2Vecs>(rd, e0, a.V, residual ? a.vec_d : a.vec_t, ld_);
        double w[PER];
        double tsum = 0.0;
        int lastpos = -1, anypos = -1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = e0 + i;
            const double xa = (double)lt_[i] - Mt;
            const double ea = exp_nonpos(xa, tab);
            double wi = ea;
            if (res) {
                const double xb = (double)ld_[i] - Md;
                const double eb = exp_nonpos(xb, tab);
                wi = (xa - xb > cls) ? fmax(ea * iS - eb * iSq, 0.0) : 0.0;
            }
            w[i] = wi;
            tsum += wi;
            if (wi > 0.0) lastpos = e;
            if (ea > 0.0) anypos = e;
        }
        double texcl;
        block_scan(tsum, scr, scan_all, &texcl);
        double cum = s_base + texcl;
        int cand = INT_MAX;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (w[i] > 0.0 && cand == INT_MAX) {
                cum += w[i];
                if (cum > target) cand = e0 + i;
            }
        }
        const int ycross = block_min_i(cand, iscr);
        const int ylast = block_max_i(lastpos, iscr);
        const int yany = block_max_i(anypos, iscr);
        if (threadIdx.x == 0) {
            s_y = ycross;
            s_ylast = ylast;
            s_yany = yany;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        // The crossing token; if rounding left none, the last token with mass
        // in the chunk; if the chunk had none, its last finite token.  Always
        // a valid index.
        int y = (s_y != INT_MAX) ? s_y : (s_ylast >= 0 ? s_ylast : s_yany);
        if (y < 0 || y >= a.V) y = 0;
        const int L = a.L;
        a.out_tok[(size_t)b * L + n] = y;
        const double lnS = log(S);
        const double ly = (double)Elem<T>::at(trow, (size_t)y);
        const double tlp = (ly - Mt) - lnS;
        double blp = tlp;
        if (res) {
            const double lnSq = log(Sq);
            const double dy = (double)Elem<T>::at(drow, (size_t)y);
            const double wy = exp_nonpos(ly - Mt, tab) * iS - exp_nonpos(dy - Md, tab) * iSq;
            const double lp = (cd.lx[n] - Mt) - lnS, lq = (cd.dx[n] - Md) - lnSq;
            const double rn = (lp == -INFINITY) ? 0.0 : exp(lp - lq);
            blp = log1p(-rn) + log(wy) - log(s_Z);
        }
        if (a.out_tlp) a.out_tlp[(size_t)b * L + n] = (float)tlp;
        if (a.out_blp) a.out_blp[(size_t)b * L + n] = (float)blp;
        ticket_reset(ticket2(a, b));
    }
    write_prefix<EXACT ? kExact : kRelaxed>(a, b, cd);
    if (threadIdx.x == 0 && s_bad_ws) a.out_status[b] = 2;
}

// ------------------------------------------------------------------- host
inline int vec_elems(spec_dtype dt) { return dt == SPEC_BF16 ? 8 : 4; }
inline int esize(spec_dtype dt) { return dt == SPEC_BF16 ? 2 : 4; }
inline int chunks(int V, int ch) { return (V + ch - 1) / ch; }
inline int tpr_of(spec_dtype dt, int V) { return chunks(V, kThreads * kTileVecs * vec_elems(dt)); }
inline int c2_of(spec_dtype dt, int V) { return chunks(V, kThreads * kP2Vecs * vec_elems(dt)); }

inline bool vec_ok(const void* p, spec_dtype dt, int V) {
    return ((uintptr_t)p % 16 == 0) && (((size_t)V * esize(dt)) % 16 == 0);
}

spec_status check_ws(void* ws, size_t bytes, int B, int R, int V, spec_dtype dt) {
    if (!ws || ((uintptr_t)ws % 256) != 0) return SPEC_EWORKSPACE;
    const Layout L = make_layout(B, R, c2_of(dt, V));
    return bytes >= L.total ? SPEC_OK : SPEC_EWORKSPACE;
}

// One-shot profiling hook: events to record around the streaming (pass-1)
// kernel of the next call made from this thread.
thread_local hipEvent_t g_prof_before = nullptr;
thread_local hipEvent_t g_prof_after = nullptr;

// Streaming grid: kWgPerCu workgroups per compute unit of the current
// device, never more workgroups than tiles.
int stream_grid(long long tiles) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    long long g = (long long)cus * kWgPerCu;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g > tiles) g = tiles;
    return (int)g;
}

// Streaming kernel, then the per-request kernel (decision, or decision and
// terminal sample).
template <int MODE, bool SUM>
spec_status launch(Args a, spec_dtype dt, hipStream_t st) {
    a.tpr = tpr_of(dt, a.V);
    a.G = stream_grid((long long)a.B * a.R * a.tpr);
    hipEvent_t before = g_prof_before, after = g_prof_after;
    g_prof_before = g_prof_after = nullptr;
    if (before && hipEventRecord(before, st) != hipSuccess) return SPEC_EHIP;
    const bool vecp = a.vec_t && (MODE != kExact || a.vec_d);
    if (dt == SPEC_BF16) {
        if (vecp)
            hipLaunchKernelGGL((k_stream<uint16_t, MODE, SUM, true>), dim3(a.G), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((k_stream<uint16_t, MODE, SUM, false>), dim3(a.G), dim3(kThreads), 0, st, a);
    } else {
        if (vecp)
            hipLaunchKernelGGL((k_stream<float, MODE, SUM, true>), dim3(a.G), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((k_stream<float, MODE, SUM, false>), dim3(a.G), dim3(kThreads), 0, st, a);
    }
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (after && hipEventRecord(after, st) != hipSuccess) return SPEC_EHIP;
    if (MODE == kGreedy || MODE == kTree) {
        if (dt == SPEC_BF16)
            hipLaunchKernelGGL((k_decide<uint16_t, MODE, SUM>), dim3(a.B), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((k_decide<float, MODE, SUM>), dim3(a.B), dim3(kThreads), 0, st, a);
    } else {
        constexpr bool EXACT = (MODE == kExact);
        const int grid = a.B * a.C2;
        if (dt == SPEC_BF16)
            hipLaunchKernelGGL((k_pass2<uint16_t, EXACT>), dim3(grid), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((k_pass2<float, EXACT>), dim3(grid), dim3(kThreads), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

bool dtype_ok(int dt) { return dt == SPEC_F32 || dt == SPEC_BF16; }

bool sizes_ok(int B, int K, int V, long rows_per_req) {
    if (B < 1 || B > kMaxB || K < 1 || V < 1 || V > SPEC_MAX_V) return false;
    // every element offset of one tensor must fit comfortably in 64 bits and
    // block counts in 31 bits
    const long long grid = (long long)B * rows_per_req * ((V + 1023) / 1024);
    return grid < (1ll << 31) && (long long)B * rows_per_req * V < (1ll << 40);
}

}  // namespace

// ============================================================== C interface
extern "C" {

size_t spec_verify_workspace_bytes(int B, int rows_per_request, int V) {
    if (B < 1 || B > kMaxB || rows_per_request < 1 || rows_per_request > kMaxRows || V < 1 ||
        V > SPEC_MAX_V)
        return 0;
    // fp32 uses the smaller chunks, so its layout bounds both dtypes
    const Layout L = make_layout(B, rows_per_request, c2_of(SPEC_F32, V));
    return L.total;
}

void spec_verify_profile_next_call(void* before_event, void* after_event) {
    g_prof_before = static_cast<hipEvent_t>(before_event);
    g_prof_after = static_cast<hipEvent_t>(after_event);
}

const char* spec_status_string(int s) {
    switch (s) {
        case SPEC_OK: return "ok";
        case SPEC_EINVAL: return "invalid argument";
        case SPEC_EDTYPE: return "unsupported dtype";
        case SPEC_EWORKSPACE: return "workspace missing, misaligned or too small";
        case SPEC_EHIP: return "HIP launch failed";
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
    if (K > SPEC_MAX_K || !sizes_ok(B, K, V, K + 1)) return SPEC_EINVAL;
    if (!target_logits || !draft_tokens || !out_tokens || !out_accept_len || !out_status)
        return SPEC_EINVAL;
    const spec_status ws = check_ws(workspace, workspace_bytes, B, K + 1, V, dtype);
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
    if (out_target_logprob) return launch<kGreedy, true>(a, dtype, st);
    return launch<kGreedy, false>(a, dtype, st);
}

spec_status spec_verify_exact(const void* target_logits, const void* draft_logits,
                              spec_dtype dtype, const int32_t* draft_tokens, const float* uniforms,
                              int B, int K, int V, int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_target_logprob, float* out_behavior_logprob,
                              int32_t* out_status, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(B, K, V, 2 * K + 1)) return SPEC_EINVAL;
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
    return launch<kExact, true>(a, dtype, st);
}

spec_status spec_verify_relaxed(const void* target_logits, spec_dtype dtype,
                                const int32_t* draft_tokens, const float* uniforms, int B, int K,
                                int V, float tau, int top_k, int32_t* out_tokens,
                                int32_t* out_accept_len, float* out_target_logprob,
                                float* out_behavior_logprob, int32_t* out_status, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (K > SPEC_MAX_K || !sizes_ok(B, K, V, K + 1)) return SPEC_EINVAL;
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
    return launch<kRelaxed, true>(a, dtype, st);
}

spec_status spec_verify_tree(const void* target_logits, spec_dtype dtype,
                             const int32_t* node_tokens, const int32_t* parents,
                             const int32_t* num_nodes, int B, int N, int V,
                             int32_t* out_path_nodes, int32_t* out_tokens, int32_t* out_accept_len,
                             float* out_target_logprob, float* out_behavior_logprob,
                             int32_t* out_status, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (N < 1 || N > SPEC_MAX_NODES || !sizes_ok(B, 1, V, N)) return SPEC_EINVAL;
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
    if (out_target_logprob) return launch<kTree, true>(a, dtype, st);
    return launch<kTree, false>(a, dtype, st);
}

}  // extern "C"
