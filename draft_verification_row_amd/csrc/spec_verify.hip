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
//           partial goes to the workspace.  An atomic ticket per request
//           elects the last workgroup of the request, which combines the
//           chunk partials of every row (fixed order, fp64), evaluates the
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
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kP1Vecs = 4;  // 16-byte vectors per thread per pass-1 chunk
constexpr int kP2Vecs = 1;  // 16-byte vectors per thread per pass-2 chunk
constexpr int kMaxRows = 2 * SPEC_MAX_K + 1;
constexpr int kMaxB = 65536;
constexpr size_t kCtrlBytes = (size_t)kMaxB * 16;  // 4 int32 per request, zero at rest

enum Mode { kGreedy = 0, kExact = 1, kRelaxed = 2, kTree = 3 };

// Chunk partial of pass 1: max, lowest index of the max, rank count and
// sum exp(l - m) over the chunk.
struct alignas(8) Part1 {
    float m;
    int idx;
    int cnt;
    int pad;
    double s;
};

// What pass 2 needs to draw the terminal token of one request.
struct alignas(8) Desc {
    int n;         // accepted drafts; the terminal token goes to position n
    int residual;  // 1: sample normalize(relu(p_n - q_n)); 0: sample p_n
    int row_t;     // absolute target row
    int row_d;     // absolute draft row (residual only)
    float Mt, Md;  // row maxima (exact)
    int pad0, pad1;
    double lnSt, lnSd;  // pass-1 log normalizers (fp32 exps, ~1e-7 relative)
    double lx, dx;      // target/draft logits at the rejected draft
};

// Chunk partial of pass 2 (fp64): sum of a = exp(l - Mt) and b = exp(d - Md)
// over the chunk, and over its tokens with p > q.
struct alignas(8) Part2 {
    double sa, sb, pa, pb;
};

struct Layout {
    size_t desc, p1, p2, total;
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline Layout make_layout(int B, int R, int C1, int C2) {
    Layout L;
    L.desc = kCtrlBytes;
    L.p1 = align_up(L.desc + (size_t)B * sizeof(Desc), 256);
    L.p2 = align_up(L.p1 + (size_t)B * R * C1 * sizeof(Part1), 256);
    L.total = align_up(L.p2 + (size_t)B * C2 * sizeof(Part2), 256);
    return L;
}

// --------------------------------------------------------------- element IO
template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bit patterns
    static constexpr int kVec = 8;
    __device__ static inline float at(const uint16_t* p, size_t i) {
        return __uint_as_float((uint32_t)p[i] << 16);
    }
    __device__ static inline void vload(const uint16_t* p, size_t i, float* v) {
        const uint4 q = *reinterpret_cast<const uint4*>(p + i);
        v[0] = __uint_as_float(q.x << 16);
        v[1] = __uint_as_float(q.x & 0xffff0000u);
        v[2] = __uint_as_float(q.y << 16);
        v[3] = __uint_as_float(q.y & 0xffff0000u);
        v[4] = __uint_as_float(q.z << 16);
        v[5] = __uint_as_float(q.z & 0xffff0000u);
        v[6] = __uint_as_float(q.w << 16);
        v[7] = __uint_as_float(q.w & 0xffff0000u);
    }
};

template <>
struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static inline float at(const float* p, size_t i) { return p[i]; }
    __device__ static inline void vload(const float* p, size_t i, float* v) {
        const float4 q = *reinterpret_cast<const float4*>(p + i);
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    }
};

// Loads vector k of this thread's share of [c0, c1): elements
// c0 + (k * kThreads + tid) * VEC + [0, VEC).  Out-of-range lanes read -inf.
template <typename T>
__device__ inline void load_vec(const T* row, long c0, long c1, int k, bool fast, float* v) {
    constexpr int VEC = Elem<T>::kVec;
    const long e0 = c0 + ((long)k * kThreads + threadIdx.x) * VEC;
    if (fast && e0 + VEC <= c1) {
        Elem<T>::vload(row, (size_t)e0, v);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            v[i] = (e0 + i < c1) ? Elem<T>::at(row, (size_t)(e0 + i)) : -INFINITY;
    }
}

// ------------------------------------------------------------ fp64 exp(x<=0)
// Cody-Waite reduction x = k ln2/64 + r, |r| <= ln2/128, then a degree-4
// Taylor polynomial (truncation error r^5/120 < 4e-14 relative) and
// 2^(k/64) = 2^(k>>6) * tab[k & 63].
constexpr double kInvLn2x64 = 92.332482616893656877;   // 64 / ln 2
constexpr double kLn2o64Hi = 0.010830424726009368896;  // ln2/64 rounded to 24 bits
constexpr double kLn2o64Lo = -2.9760223436840126e-11;  // ln2/64 - hi

__device__ inline double exp_nonpos(double x, const double* tab) {
    if (!(x > -700.0)) return 0.0;
    const double kd = __builtin_rint(x * kInvLn2x64);
    const int k = (int)kd;
    double r = fma(-kd, kLn2o64Hi, x);
    r = fma(-kd, kLn2o64Lo, r);
    double p = fma(r, 1.0 / 24.0, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    return ldexp(tab[k & 63] * p, k >> 6);
}

__device__ inline void fill_exp_table(double* tab) {
    if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
}

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ wave helpers
__device__ inline void argmax_combine(float& m, int& idx, float om, int oi) {
    if (om > m || (om == m && oi < idx)) {
        m = om;
        idx = oi;
    }
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ inline int wave_sum_i(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
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
    int C1, C2;  // chunks per row in pass 1 / pass 2
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

__device__ inline int* ticket1(const Args& a, int b) { return reinterpret_cast<int*>(a.ws) + 4 * b; }
__device__ inline int* ticket2(const Args& a, int b) {
    return reinterpret_cast<int*>(a.ws) + 4 * b + 1;
}

// -------------------------------------------------------------------- pass 1
template <typename T, int MODE, bool SUM>
__global__ __launch_bounds__(kThreads) void k_pass1(const Args a) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int CH = kThreads * kP1Vecs * VEC;
    constexpr bool ARGMAX = (MODE == kGreedy || MODE == kTree);
    constexpr bool COUNT = (MODE == kRelaxed);

    const Layout lay = make_layout(a.B, a.R, a.C1, a.C2);
    Part1* part = reinterpret_cast<Part1*>(a.ws + lay.p1);
    Desc* desc = reinterpret_cast<Desc*>(a.ws + lay.desc);

    const int bid = blockIdx.x;
    const int c = bid % a.C1;
    const int rr = (bid / a.C1) % a.R;
    const int b = bid / (a.C1 * a.R);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    int nb = a.rows_t;
    if (MODE == kTree && a.num_nodes) nb = min(max(a.num_nodes[b], 1), a.rows_t);

    const T* row;
    bool fast;
    if (MODE == kExact && rr >= a.rows_t) {
        row = reinterpret_cast<const T*>(a.D) + (size_t)(b * a.K + (rr - a.rows_t)) * a.V;
        fast = a.vec_d;
    } else {
        row = reinterpret_cast<const T*>(a.T) + (size_t)(b * a.rows_t + rr) * a.V;
        fast = a.vec_t;
    }
    const bool active = (MODE != kTree) || rr < nb;
    float thr = INFINITY;
    if (COUNT && rr < a.K) {
        const int x = a.tok[b * a.K + rr];
        if ((unsigned)x < (unsigned)a.V) thr = Elem<T>::at(row, (size_t)x);
    }

    __shared__ float s_m[kWaves];
    __shared__ int s_i[kWaves];
    __shared__ int s_c[kWaves];
    __shared__ double s_s[kWaves];
    __shared__ int s_last;

    if (active) {
        const long c0 = (long)c * CH;
        const long c1 = min(c0 + (long)CH, (long)a.V);
        float v[kP1Vecs][VEC];
#pragma unroll
        for (int k = 0; k < kP1Vecs; ++k) load_vec<T>(row, c0, c1, k, fast, v[k]);

        float m = -INFINITY;
        int idx = INT_MAX;
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kP1Vecs; ++k) {
            const int base = (int)(c0 + ((long)k * kThreads + threadIdx.x) * VEC);
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                if (ARGMAX) {
                    if (v[k][i] > m) {
                        m = v[k][i];
                        idx = base + i;
                    }
                } else {
                    m = fmaxf(m, v[k][i]);
                }
                if (COUNT) cnt += (v[k][i] > thr) ? 1 : 0;
            }
        }
        // wave max (and lowest-index argmax)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float om = __shfl_xor(m, off);
            if (ARGMAX) {
                const int oi = __shfl_xor(idx, off);
                argmax_combine(m, idx, om, oi);
            } else {
                m = fmaxf(m, om);
            }
        }
        double s = 0.0;
        if (SUM && m > -INFINITY) {
#pragma unroll
            for (int k = 0; k < kP1Vecs; ++k) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    acc += __builtin_amdgcn_exp2f((v[k][i] - m) * kLog2e);
                s += (double)acc;
            }
            s = wave_sum(s);
        }
        if (COUNT) cnt = wave_sum_i(cnt);
        if (lane == 0) {
            s_m[wave] = m;
            s_i[wave] = idx;
            s_c[wave] = cnt;
            s_s[wave] = s;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float M = s_m[0];
            int I = s_i[0];
            for (int w = 1; w < kWaves; ++w) argmax_combine(M, I, s_m[w], s_i[w]);
            double S = 0.0;
            int C = 0;
            for (int w = 0; w < kWaves; ++w) {
                if (SUM && s_m[w] > -INFINITY) S += s_s[w] * exp((double)s_m[w] - (double)M);
                C += s_c[w];
            }
            Part1 p;
            p.m = M;
            p.idx = I;
            p.cnt = C;
            p.pad = 0;
            p.s = S;
            part[bid] = p;
        }
    }

    // elect the last workgroup of this request
    if (threadIdx.x == 0) {
        __threadfence();
        const int prev = atomicAdd(ticket1(a, b), 1);
        s_last = (prev == a.R * a.C1 - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // ---- per-request decision (last workgroup only)
    __shared__ float r_M[kMaxRows];
    __shared__ int r_g[kMaxRows];
    __shared__ int r_c[kMaxRows];
    __shared__ double r_lnS[kMaxRows];

    const int rows_used = (MODE == kTree) ? nb : a.R;
    for (int r = threadIdx.x; r < rows_used; r += kThreads) {
        const Part1* pr = part + (size_t)(b * a.R + r) * a.C1;
        float M = -INFINITY;
        int g = INT_MAX;
        int C = 0;
        for (int cc = 0; cc < a.C1; ++cc) {
            const Part1 p = pr[cc];
            argmax_combine(M, g, p.m, p.idx);
            C += p.cnt;
        }
        double S = 0.0;
        if (SUM && M > -INFINITY)
            for (int cc = 0; cc < a.C1; ++cc) {
                const Part1 p = pr[cc];
                if (p.m > -INFINITY) S += p.s * exp((double)p.m - (double)M);
            }
        r_M[r] = M;
        r_g[r] = g;
        r_c[r] = C;
        r_lnS[r] = log(S);
    }
    __syncthreads();

    const T* Tp = reinterpret_cast<const T*>(a.T);
    const T* Dp = reinterpret_cast<const T*>(a.D);
    const int K = a.K;
    const int L = a.L;

    if (MODE == kGreedy || MODE == kExact || MODE == kRelaxed) {
        if (wave == 0) {
            const int j = lane;
            bool acc = false, bad = false;
            int x = -1;
            double lp = 0.0, lq = 0.0, lx = -INFINITY, dx = -INFINITY;
            if (j < K) {
                x = a.tok[b * K + j];
                bad = (unsigned)x >= (unsigned)a.V;
                if (!bad) {
                    if (MODE == kGreedy) {
                        acc = (x == r_g[j]);
                        lp = -r_lnS[j];
                    } else {
                        lx = Elem<T>::at(Tp, (size_t)(b * a.rows_t + j) * a.V + x);
                        lp = (lx - (double)r_M[j]) - r_lnS[j];
                        if (MODE == kExact) {
                            dx = Elem<T>::at(Dp, (size_t)(b * K + j) * a.V + x);
                            lq = (dx - (double)r_M[a.rows_t + j]) - r_lnS[a.rows_t + j];
                            double r;
                            if (lp == -INFINITY)
                                r = 0.0;
                            else if (lq == -INFINITY)
                                r = INFINITY;
                            else
                                r = exp(lp - lq);
                            acc = (double)a.u[b * (K + 1) + j] < r;
                        } else {
                            acc = (r_c[j] < a.top_k) || (exp(lp) >= (double)a.tau);
                        }
                    }
                }
            }
            const unsigned long long mask = __ballot(acc);
            const int n = __builtin_ctzll(~mask);  // lane K never accepts, so n <= K
            int32_t* otok = a.out_tok + (size_t)b * L;
            float* otlp = a.out_tlp ? a.out_tlp + (size_t)b * L : nullptr;
            float* oblp = a.out_blp ? a.out_blp + (size_t)b * L : nullptr;
            if (j < n) {
                otok[j] = x;
                if (otlp) otlp[j] = (float)lp;
                if (oblp) oblp[j] = (MODE == kExact) ? (float)fmin(0.0, lp - lq) : 0.f;
            } else if (j > n && j < L) {
                otok[j] = -1;
                if (otlp) otlp[j] = 0.f;
                if (oblp) oblp[j] = 0.f;
            } else if (j == n) {
                a.out_len[b] = n;
                a.out_status[b] = (n < K && bad) ? 1 : 0;
                if (MODE == kGreedy) {
                    otok[n] = r_g[n];
                    if (otlp) otlp[n] = (float)(-r_lnS[n]);
                    if (oblp) oblp[n] = 0.f;
                } else {
                    Desc d;
                    d.n = n;
                    d.residual = (MODE == kExact && n < K) ? 1 : 0;
                    d.row_t = b * a.rows_t + n;
                    d.row_d = b * K + n;
                    d.Mt = r_M[n];
                    d.lnSt = r_lnS[n];
                    d.Md = d.residual ? r_M[a.rows_t + n] : 0.f;
                    d.lnSd = d.residual ? r_lnS[a.rows_t + n] : 0.0;
                    d.lx = lx;
                    d.dx = dx;
                    d.pad0 = d.pad1 = 0;
                    desc[b] = d;
                }
            }
        }
    } else {  // tree
        __shared__ int t_par[SPEC_MAX_NODES];
        __shared__ int t_match[SPEC_MAX_NODES];
        __shared__ int t_path[SPEC_MAX_NODES];
        __shared__ int t_d, t_e, t_bad;
        const int N = a.rows_t;
        if (wave == 0) {
            const int i = lane;
            bool bad = false;
            if (i >= 1 && i < nb) {
                const int p = a.parents[b * N + i];
                const int t = a.tok[b * N + i];
                bad = !(p >= 0 && p < i && (unsigned)t < (unsigned)a.V);
                t_par[i] = bad ? -1 : p;
                t_match[i] = bad ? 0 : (t == r_g[p]);
            }
            const unsigned long long bm = __ballot(bad);
            if (lane == 0) t_bad = bm != 0ull;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            // accepted iff matched and parent accepted; parents precede children
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
                if (a.out_tlp) a.out_tlp[(size_t)b * N + k] = (float)(-r_lnS[t_par[v]]);
            } else {
                a.out_path[(size_t)b * N + k] = -1;
                otok[k] = (k == d) ? r_g[e] : -1;
                if (a.out_tlp) a.out_tlp[(size_t)b * N + k] = (k == d) ? (float)(-r_lnS[e]) : 0.f;
            }
            if (a.out_blp) a.out_blp[(size_t)b * N + k] = 0.f;
        }
        if (threadIdx.x == 0) {
            a.out_len[b] = d;
            a.out_status[b] = t_bad;
        }
    }
    if (threadIdx.x == 0) *ticket1(a, b) = 0;
}

// -------------------------------------------------------------------- pass 2
template <typename T, bool EXACT>
__global__ __launch_bounds__(kThreads) void k_pass2(const Args a) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int CH = kThreads * kP2Vecs * VEC;
    const Layout lay = make_layout(a.B, a.R, a.C1, a.C2);
    Part2* part = reinterpret_cast<Part2*>(a.ws + lay.p2);
    const Desc* descs = reinterpret_cast<const Desc*>(a.ws + lay.desc);

    const int b = blockIdx.x / a.C2;
    const int c = blockIdx.x % a.C2;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    __shared__ double tab[64];
    __shared__ double red[kWaves][4];
    __shared__ int s_last;
    fill_exp_table(tab);
    __syncthreads();

    const Desc d = descs[b];
    const bool residual = EXACT && d.residual;
    const T* trow = reinterpret_cast<const T*>(a.T) + (size_t)d.row_t * a.V;
    const T* drow = reinterpret_cast<const T*>(a.D) + (size_t)d.row_d * a.V;
    const double Mt = d.Mt, Md = d.Md;
    const double cls = d.lnSt - d.lnSd;  // p > q  <=>  (l - Mt) - (d - Md) > lnSt - lnSd

    const long c0 = (long)c * CH;
    const long c1 = min(c0 + (long)CH, (long)a.V);
    double sa = 0.0, sb = 0.0, pa = 0.0, pb = 0.0;
#pragma unroll
    for (int k = 0; k < kP2Vecs; ++k) {
        float vt[VEC], vd[VEC];
        load_vec<T>(trow, c0, c1, k, a.vec_t, vt);
        if (residual) load_vec<T>(drow, c0, c1, k, a.vec_d, vd);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const double xa = (double)vt[i] - Mt;
            const double ea = exp_nonpos(xa, tab);
            sa += ea;
            if (residual) {
                const double xb = (double)vd[i] - Md;
                const double eb = exp_nonpos(xb, tab);
                sb += eb;
                if (xa - xb > cls) {
                    pa += ea;
                    pb += eb;
                }
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
        Part2 p = {0.0, 0.0, 0.0, 0.0};
        for (int w = 0; w < kWaves; ++w) {
            p.sa += red[w][0];
            p.sb += red[w][1];
            p.pa += red[w][2];
            p.pb += red[w][3];
        }
        part[(size_t)b * a.C2 + c] = p;
        __threadfence();
        const int prev = atomicAdd(ticket2(a, b), 1);
        s_last = (prev == a.C2 - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // ---- terminal sample (last workgroup of the request)
    __shared__ double s_S, s_Sq, s_Z, s_base, s_target;
    __shared__ int s_cstar, s_res;
    __shared__ int s_y, s_ylast, s_yany;
    const Part2* pr = part + (size_t)b * a.C2;
    if (threadIdx.x == 0) {
        double S = 0.0, Sq = 0.0;
        for (int cc = 0; cc < a.C2; ++cc) {
            S += pr[cc].sa;
            Sq += pr[cc].sb;
        }
        bool res = residual;
        double Z = 0.0;
        if (res) {
            for (int cc = 0; cc < a.C2; ++cc) Z += pr[cc].pa / S - pr[cc].pb / Sq;
            if (!(Z > 0.0)) res = false;
        }
        if (!res) Z = S;
        const double target = (double)a.u[b * (a.K + 1) + a.K] * Z;
        double cum = 0.0, base_last = 0.0;
        int cstar = -1, clast = 0;
        for (int cc = 0; cc < a.C2; ++cc) {
            const double W = res ? (pr[cc].pa / S - pr[cc].pb / Sq) : pr[cc].sa;
            if (!(W > 0.0)) continue;
            if (cum + W > target) {
                cstar = cc;
                break;
            }
            clast = cc;
            base_last = cum;
            cum += W;
        }
        if (cstar < 0) {  // rounding: fall back to the last chunk with mass
            cstar = clast;
            cum = base_last;
        }
        s_S = S;
        s_Sq = Sq;
        s_Z = Z;
        s_res = res;
        s_base = cum;
        s_target = target;
        s_cstar = cstar;
        s_y = INT_MAX;
        s_ylast = -1;
        s_yany = -1;
    }
    __syncthreads();
    const bool res = s_res;
    const double S = s_S, Sq = s_Sq;
    const double target = s_target;
    {
        const long e0c = (long)s_cstar * CH;
        const long e1c = min(e0c + (long)CH, (long)a.V);
        double w[kP2Vecs * VEC];
        double tsum = 0.0;
        int lastpos = -1, anypos = -1;
#pragma unroll
        for (int k = 0; k < kP2Vecs; ++k) {
            float vt[VEC], vd[VEC];
            load_vec<T>(trow, e0c, e1c, k, a.vec_t, vt);
            if (res) load_vec<T>(drow, e0c, e1c, k, a.vec_d, vd);
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const double xa = (double)vt[i] - Mt;
                const double ea = exp_nonpos(xa, tab);
                double wi;
                if (res) {
                    const double xb = (double)vd[i] - Md;
                    const double eb = exp_nonpos(xb, tab);
                    wi = (xa - xb > cls) ? fmax(ea / S - eb / Sq, 0.0) : 0.0;
                } else {
                    wi = ea;
                }
                w[k * VEC + i] = wi;
                tsum += wi;
                const int pos = (int)(e0c + ((long)k * kThreads + threadIdx.x) * VEC + i);
                if (wi > 0.0) lastpos = pos;
                if (ea > 0.0) anypos = pos;
            }
        }
        // exclusive scan of per-thread sums in thread order.  With
        // kP2Vecs == 1 each thread owns one contiguous run of VEC tokens, so
        // thread order is token order.
        static_assert(kP2Vecs == 1, "in-chunk scan assumes one vector per thread");
        double incl = tsum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        __shared__ double wtot[kWaves];
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        double excl = s_base + (incl - tsum);
        for (int ww = 0; ww < wave; ++ww) excl += wtot[ww];
        double cum = excl;
        int cand = INT_MAX;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            if (w[i] > 0.0) {
                cum += w[i];
                if (cum > target) {
                    cand = (int)(e0c + (long)threadIdx.x * VEC + i);
                    break;
                }
            }
        }
        if (cand != INT_MAX) atomicMin(&s_y, cand);
        if (lastpos >= 0) atomicMax(&s_ylast, lastpos);
        if (anypos >= 0) atomicMax(&s_yany, anypos);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        // The crossing token; if rounding left none, the last token with mass
        // in the chunk; if the chunk had none, its last finite token.  Always
        // a valid index.
        int y = (s_y != INT_MAX) ? s_y : (s_ylast >= 0 ? s_ylast : s_yany);
        if (y < 0 || y >= a.V) y = 0;
        const int n = d.n;
        const int L = a.L;
        a.out_tok[(size_t)b * L + n] = y;
        const double lnS = log(S);
        const double ly = (double)Elem<T>::at(trow, (size_t)y);
        const double tlp = (ly - Mt) - lnS;
        double blp = tlp;
        if (res) {
            const double lnSq = log(Sq);
            const double dy = (double)Elem<T>::at(drow, (size_t)y);
            const double wy = exp_nonpos(ly - Mt, tab) / S - exp_nonpos(dy - Md, tab) / Sq;
            const double lp = (d.lx - Mt) - lnS, lq = (d.dx - Md) - lnSq;
            const double rn = (lp == -INFINITY) ? 0.0 : exp(lp - lq);
            blp = log1p(-rn) + log(wy) - log(s_Z);
        }
        if (a.out_tlp) a.out_tlp[(size_t)b * L + n] = (float)tlp;
        if (a.out_blp) a.out_blp[(size_t)b * L + n] = (float)blp;
        *ticket2(a, b) = 0;
    }
}

// ------------------------------------------------------------------- host
inline int vec_elems(spec_dtype dt) { return dt == SPEC_BF16 ? 8 : 4; }
inline int esize(spec_dtype dt) { return dt == SPEC_BF16 ? 2 : 4; }
inline int chunks(int V, int ch) { return (V + ch - 1) / ch; }
inline int c1_of(spec_dtype dt, int V) { return chunks(V, kThreads * kP1Vecs * vec_elems(dt)); }
inline int c2_of(spec_dtype dt, int V) { return chunks(V, kThreads * kP2Vecs * vec_elems(dt)); }

inline bool vec_ok(const void* p, spec_dtype dt, int V) {
    return ((uintptr_t)p % 16 == 0) && (((size_t)V * esize(dt)) % 16 == 0);
}

spec_status check_ws(void* ws, size_t bytes, int B, int R, int V, spec_dtype dt) {
    if (!ws || ((uintptr_t)ws % 256) != 0) return SPEC_EWORKSPACE;
    const Layout L = make_layout(B, R, c1_of(dt, V), c2_of(dt, V));
    return bytes >= L.total ? SPEC_OK : SPEC_EWORKSPACE;
}

template <int MODE, bool SUM>
spec_status launch_p1(const Args& a, spec_dtype dt, hipStream_t st) {
    const int grid = a.B * a.R * a.C1;
    if (dt == SPEC_BF16)
        hipLaunchKernelGGL((k_pass1<uint16_t, MODE, SUM>), dim3(grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_pass1<float, MODE, SUM>), dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

template <bool EXACT>
spec_status launch_p2(const Args& a, spec_dtype dt, hipStream_t st) {
    const int grid = a.B * a.C2;
    if (dt == SPEC_BF16)
        hipLaunchKernelGGL((k_pass2<uint16_t, EXACT>), dim3(grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_pass2<float, EXACT>), dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

bool dtype_ok(int dt) { return dt == SPEC_F32 || dt == SPEC_BF16; }

bool sizes_ok(int B, int K, int V, long rows_per_req) {
    if (B < 1 || B > kMaxB || K < 1 || V < 1) return false;
    // every element offset of one tensor must fit comfortably in 64 bits and
    // block counts in 31 bits
    const long long grid = (long long)B * rows_per_req * ((V + 1023) / 1024);
    return grid < (1ll << 31) && (long long)B * rows_per_req * V < (1ll << 40);
}

}  // namespace

// ============================================================== C interface
extern "C" {

size_t spec_verify_workspace_bytes(int B, int rows_per_request, int V) {
    if (B < 1 || B > kMaxB || rows_per_request < 1 || rows_per_request > kMaxRows || V < 1) return 0;
    // fp32 uses the smaller chunks, so its layout bounds both dtypes
    const Layout L = make_layout(B, rows_per_request, c1_of(SPEC_F32, V), c2_of(SPEC_F32, V));
    return L.total;
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
    a.C1 = c1_of(dtype, V);
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
    if (out_target_logprob) return launch_p1<kGreedy, true>(a, dtype, st);
    return launch_p1<kGreedy, false>(a, dtype, st);
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
    a.C1 = c1_of(dtype, V);
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
    spec_status s = launch_p1<kExact, true>(a, dtype, st);
    if (s != SPEC_OK) return s;
    return launch_p2<true>(a, dtype, st);
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
    a.C1 = c1_of(dtype, V);
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
    spec_status s = launch_p1<kRelaxed, true>(a, dtype, st);
    if (s != SPEC_OK) return s;
    return launch_p2<false>(a, dtype, st);
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
    a.C1 = c1_of(dtype, V);
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
    if (out_target_logprob) return launch_p1<kTree, true>(a, dtype, st);
    return launch_p1<kTree, false>(a, dtype, st);
}

}  // extern "C"
