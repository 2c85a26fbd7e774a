// sv_verify.hip -- batched speculative-decoding verification for MI355X
// (gfx950, CDNA4, wave64).
//
// What is computed: the verification step of the spec-verify kernel card
// (section "Method", greedy and speculative-sampling bullets; unnormalised
// masses from its "Correctness" section).  Conventions where the card is
// silent are stated in include/sv_verify.h.
//
// Work decomposition (the vocabulary axis is the long one):
//   * every row of V values is cut into NC = ceil(V / 8192) chunks; a
//     256-thread block (4 waves) owns one chunk of one row; each thread loads
//     8 float4 per operand (coalesced 16-byte loads, 32 KB per operand per
//     block) and keeps them in VGPRs;
//   * per-chunk partials (fp64 masses, lowest-index argmax) are combined per
//     row by the last block to arrive (agent-scope acq_rel ticket), always in
//     the same lane order, so every result depends on V alone, never on B, K,
//     the launch shape or timing;
//   * greedy needs nothing more: the last row of a sequence to complete
//     resolves (n_accepted, next_token);
//   * sampled runs persistently with atomic work tickets handed out in
//     (sequence, row, chunk) order.  After its row has been combined every
//     block of a rejecting row computes its chunk's residual mass from the
//     values still in registers; after a second row-level rendezvous the one
//     block whose chunk holds u_K * W runs the inverse-CDF search in
//     registers.  The bonus row works the same way on the mass partials.  No
//     row is read twice from HBM.
//
// Deadlock freedom of the row rendezvous: tickets are taken in order, so all
// rows except the one holding the newest ticket have every chunk taken, and
// their blocks reach the rendezvous without waiting.  A block waits only on
// its own row, so at most NC - 1 blocks wait on the one incomplete row; the
// host launches at least NC resident blocks, so some block always advances.
// Every wait is also bounded (it raises the workspace fault word instead of
// spinning forever).

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "sv_verify.h"

#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVec = 8;                        // float4 per thread per operand
constexpr int kChunk4 = kThreads * kVec;       // float4 per chunk
constexpr int kChunk = kChunk4 * 4;            // 8192 values per chunk
constexpr int kMaxChunks = 64;                 // one chunk per lane of a wave
static_assert(SV_MAX_V == kMaxChunks * kChunk, "SV_MAX_V must match the chunk geometry");
constexpr double kWaitSeconds = 2.0;           // bound of every cross-block wait

struct Header {              // 256 bytes
    unsigned ticket;         // next work ticket (sampled)
    unsigned exit_count;     // blocks that left the ticket loop (sampled)
    unsigned error;          // sticky fault word: a bounded wait expired
    unsigned pad[61];
};

struct ChunkPart {           // 32 bytes
    double sp, sq, smin;     // chunk sums of p, q, min(p, q)
    float maxv;
    int arg;
};

struct RowRes {              // 64 bytes
    double P, Q, Smin, W;
    float maxv, pt, qt;
    int arg;
    int acc, draw, cand, pad;
};

struct Layout {
    size_t hdr, cnt1, cnt2, flag1, flag2, seqcnt, rowres, parts, wpart, prefp, prefw, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline Layout make_layout(int64_t B, int64_t K, int64_t NC)
{
    const size_t R = (size_t)(B * (K + 1));
    Layout L{};
    size_t o = 0;
    L.hdr = o;    o = align_up(o + sizeof(Header), 256);
    L.cnt1 = o;   o = align_up(o + R * 4, 256);
    L.cnt2 = o;   o = align_up(o + R * 4, 256);
    L.flag1 = o;  o = align_up(o + R * 4, 256);
    L.flag2 = o;  o = align_up(o + R * 4, 256);
    L.seqcnt = o; o = align_up(o + (size_t)B * 4, 256);
    L.rowres = o; o = align_up(o + R * sizeof(RowRes), 256);
    L.parts = o;  o = align_up(o + R * (size_t)NC * sizeof(ChunkPart), 256);
    L.wpart = o;  o = align_up(o + R * (size_t)NC * 8, 256);
    L.prefp = o;  o = align_up(o + R * (size_t)(NC + 1) * 8, 256);
    L.prefw = o;  o = align_up(o + R * (size_t)(NC + 1) * 8, 256);
    L.total = o;
    return L;
}

struct Args {
    const float* tp;
    const float* dp;
    const int32_t* dt;
    const float* u;
    int32_t* n_out;
    int32_t* next_out;
    sv_row_stats* stats;
    Header* hdr;
    unsigned *cnt1, *cnt2, *flag1, *flag2, *seqcnt;
    RowRes* rowres;
    ChunkPart* parts;
    double* wpart;
    double* prefp;
    double* prefw;
    int B, K, V, NC;
    unsigned total;          // work items (sampled)
    unsigned long long wait_ticks;   // wait bound in wall-clock ticks
};

// ------------------------------------------- cross-block communication --
//
// Every value one block publishes for another (chunk partials, row results,
// prefixes, counters, flags) is written and read with agent-scope atomic
// accesses.  On gfx950 these are performed at the device-coherent level
// (sc1 loads and stores; RMW atomics at the memory side) instead of in the
// per-XCD L2, so no L2 write-back or invalidate (the cost of agent-scope
// release/acquire fences) is ever needed.  Ordering is explicit:
//   writer: data stores -> publish() -> counter RMW or flag store
//   reader: counter RMW or flag load -> observe() -> data loads
// publish() waits for the wave's outstanding memory operations to complete
// (gfx9 counts stores in vmcnt); both are compiler barriers.

__device__ __forceinline__ void publish() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void observe() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ unsigned count_up(unsigned* p)
{
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_u32(void* p, unsigned v)
{
    __hip_atomic_store(static_cast<unsigned*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned get_u32(const void* p)
{
    return __hip_atomic_load(static_cast<const unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_u64(void* p, unsigned long long v)
{
    __hip_atomic_store(static_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_u64(const void* p)
{
    return __hip_atomic_load(static_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_i32(int* p, int v) { put_u32(p, (unsigned)v); }
__device__ __forceinline__ int get_i32(const int* p) { return (int)get_u32(p); }
__device__ __forceinline__ void put_f32(float* p, float v) { put_u32(p, __float_as_uint(v)); }
__device__ __forceinline__ float get_f32(const float* p) { return __uint_as_float(get_u32(p)); }
__device__ __forceinline__ void put_f64(double* p, double v)
{
    put_u64(p, (unsigned long long)__double_as_longlong(v));
}
__device__ __forceinline__ double get_f64(const double* p)
{
    return __longlong_as_double((long long)get_u64(p));
}

// Bounded wait for a row flag; on expiry raises the fault word and returns
// (the call's outputs are then unspecified, but every block still exits).
__device__ __forceinline__ void wait_flag(const unsigned* flag, Header* hdr, unsigned long long ticks)
{
    const unsigned long long t0 = wall_clock64();
    while (get_u32(flag) == 0u) {
        __builtin_amdgcn_s_sleep(2);
        if (wall_clock64() - t0 > ticks) {
            put_u32(&hdr->error, 1u);
            break;
        }
    }
    observe();
}

// Wave-cooperative zeroing of [p, p + bytes), p 8-byte aligned, bytes % 8 == 0.
__device__ __forceinline__ void wave_zero(void* p, size_t bytes)
{
    unsigned long long* q = static_cast<unsigned long long*>(p);
    const size_t n = bytes / 8;
    for (size_t j = threadIdx.x & 63; j < n; j += 64) put_u64(q + j, 0ull);
}

// Once sequence b is resolved nothing reads its partials, prefixes or row
// results again: return them to zero so that the whole workspace is zero
// between calls, whatever shapes the next call uses.
__device__ __forceinline__ void zero_sequence_data(const Args& a, int b, bool sampled)
{
    const int64_t rows = a.K + 1, r0 = (int64_t)b * rows, NC = a.NC;
    wave_zero(a.parts + r0 * NC, (size_t)(rows * NC) * sizeof(ChunkPart));
    wave_zero(a.rowres + r0, (size_t)rows * sizeof(RowRes));
    if (sampled) {
        wave_zero(a.wpart + r0 * NC, (size_t)(rows * NC) * 8);
        wave_zero(a.prefp + r0 * (NC + 1), (size_t)(rows * (NC + 1)) * 8);
        wave_zero(a.prefw + r0 * (NC + 1), (size_t)(rows * (NC + 1)) * 8);
    }
}

// ---------------------------------------------------------- chunk I/O --

// Thread t holds float4 number (c * kChunk4 + k * 256 + t) of the row, k < 8:
// consecutive threads read consecutive 16-byte words (fully coalesced).
__device__ __forceinline__ int f4_index(int c, int k) { return c * kChunk4 + k * kThreads + (int)threadIdx.x; }

template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int V, int c, float4 (&v)[kVec])
{
    if constexpr (VEC) {
        const float4* r4 = reinterpret_cast<const float4*>(row);
        const int nf = V >> 2;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const int f = f4_index(c, k);
            v[k] = f < nf ? r4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const int x = f4_index(c, k) * 4;
            v[k].x = x + 0 < V ? row[x + 0] : 0.f;
            v[k].y = x + 1 < V ? row[x + 1] : 0.f;
            v[k].z = x + 2 < V ? row[x + 2] : 0.f;
            v[k].w = x + 3 < V ? row[x + 3] : 0.f;
        }
    }
}

// Opaque to the optimiser: forces later phases to reconvert the f32 values
// kept in registers instead of keeping fp64 copies of all of them alive.
__device__ __forceinline__ void reg_barrier(float4 (&v)[kVec])
{
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        float x = v[k].x, y = v[k].y, z = v[k].z, w = v[k].w;
        asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
        v[k] = make_float4(x, y, z, w);
    }
}

__device__ __forceinline__ float comp(float4 v, int e)
{
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// ------------------------------------------------------- reductions --

struct Acc {
    double sp, sq, smin;
    float maxv;
    int arg;
};

// (value, index) order: larger value first, then lower index (lowest-index
// argmax).  A total order, so any merge tree gives the same result.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi)
{
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

template <bool PAIR>
__device__ __forceinline__ Acc thread_stats(const float4 (&pv)[kVec], const float4 (&qv)[kVec], int V, int c)
{
    Acc a{0.0, 0.0, 0.0, -INFINITY, INT_MAX};
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        const int x0 = f4_index(c, k) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = comp(pv[k], e);
            if (x0 + e < V && p > a.maxv) {
                a.maxv = p;
                a.arg = x0 + e;
            }
            a.sp += (double)p;                       // padding values are 0
            if constexpr (PAIR) {
                const float q = comp(qv[k], e);
                a.sq += (double)q;
                a.smin += (double)fminf(p, q);
            }
        }
    }
    return a;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;   // identical in every lane (each level adds the same pair)
}

__device__ __forceinline__ double wave_inclusive_scan(double v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double y = __shfl_up(v, d);
        if (lane >= d) v += y;
    }
    return v;
}

// Block reduction; the result is valid in thread 0.
template <bool PAIR>
__device__ __forceinline__ Acc block_reduce(Acc a)
{
    __shared__ double s_sp[kWaves], s_sq[kWaves], s_sm[kWaves];
    __shared__ float s_v[kWaves];
    __shared__ int s_i[kWaves];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a.sp += __shfl_xor(a.sp, off);
        if constexpr (PAIR) {
            a.sq += __shfl_xor(a.sq, off);
            a.smin += __shfl_xor(a.smin, off);
        }
        const float ov = __shfl_xor(a.maxv, off);
        const int oi = __shfl_xor(a.arg, off);
        argmax_merge(a.maxv, a.arg, ov, oi);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        s_sp[w] = a.sp;
        s_sq[w] = a.sq;
        s_sm[w] = a.smin;
        s_v[w] = a.maxv;
        s_i[w] = a.arg;
    }
    __syncthreads();
    Acc r = a;
    if (threadIdx.x == 0) {
        r = Acc{s_sp[0], s_sq[0], s_sm[0], s_v[0], s_i[0]};
        for (int j = 1; j < kWaves; ++j) {
            r.sp += s_sp[j];
            r.sq += s_sq[j];
            r.smin += s_sm[j];
            argmax_merge(r.maxv, r.arg, s_v[j], s_i[j]);
        }
    }
    return r;
}

__device__ __forceinline__ double block_sum(double v)
{
    __shared__ double s[kWaves];
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = v;
    if (threadIdx.x == 0) {
        r = s[0];
        for (int j = 1; j < kWaves; ++j) r += s[j];
    }
    return r;
}

// ------------------------------------------------------ row combine --

// Wave 0 of the block that completed a row: combine the NC chunk partials in
// lane (= chunk) order, publish the row result, the prefix of the chunk mass
// partials and, when `stats` is set, the row statistics; then release the
// row flag (sampled) so the other chunks of the row may proceed.
template <bool SAMPLED>
__device__ __forceinline__ void combine_row(const Args& a, int b, int i, int64_t row)
{
    const int lane = threadIdx.x & 63;
    const int NC = a.NC, K = a.K, V = a.V;
    const bool pair = SAMPLED && i < K;
    observe();
    ChunkPart cp{0.0, 0.0, 0.0, -INFINITY, INT_MAX};
    if (lane < NC) {
        const ChunkPart* src = &a.parts[row * NC + lane];
        cp.sp = get_f64(&src->sp);
        if (pair) {
            cp.sq = get_f64(&src->sq);
            cp.smin = get_f64(&src->smin);
        }
        cp.maxv = get_f32(&src->maxv);
        cp.arg = get_i32(&src->arg);
    }
    float mv = cp.maxv;
    int ai = cp.arg;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(mv, off);
        const int oi = __shfl_xor(ai, off);
        argmax_merge(mv, ai, ov, oi);
    }
    const double incl = wave_inclusive_scan(cp.sp);
    const double P = __shfl(incl, NC - 1);
    double Q = 0.0, Smin = 0.0;
    if (pair) {
        Q = wave_sum(cp.sq);
        Smin = wave_sum(cp.smin);
    }
    if (SAMPLED) {
        double* pref = a.prefp + row * (NC + 1);
        if (lane < NC) put_f64(&pref[lane + 1], incl);
        if (lane == 0) put_f64(&pref[0], 0.0);
    }
    if (lane == 0) {
        const int t = i < K ? a.dt[(int64_t)b * K + i] : -1;
        const bool tin = t >= 0 && t < V;
        const float pt = (i < K && tin) ? a.tp[row * V + t] : 0.0f;
        const float qt = (pair && tin) ? a.dp[((int64_t)b * K + i) * V + t] : 0.0f;
        int acc = 1, draw = SAMPLED ? 1 : 0;
        if (pair) {
            const double ui = (double)a.u[(int64_t)b * (K + 1) + i];
            acc = (ui * (double)qt * P < (double)pt * Q) ? 1 : 0;
            draw = acc ? 0 : 1;
        }
        RowRes* rr = &a.rowres[row];
        put_f64(&rr->P, P);
        put_f64(&rr->Q, Q);
        put_i32(&rr->arg, ai);
        put_i32(&rr->acc, acc);
        put_i32(&rr->draw, draw);
        put_i32(&rr->cand, -1);
        if (a.stats) {
            sv_row_stats s;
            s.argmax = ai;
            s.max_p = mv;
            s.sum_p = P;
            s.sum_q = Q;
            s.sum_min = Smin;
            s.sum_pos = pair ? P - Smin : 0.0;
            s.p_t = pt;
            s.q_t = qt;
            a.stats[row] = s;
        }
        put_u32(&a.cnt1[row], 0u);           // nobody else touches it this launch
        publish();
        if (SAMPLED) put_u32(&a.flag1[row], 1u);
    }
}

// Wave 0 of the block that completed the residual partials of a row.
__device__ __forceinline__ void combine_residual(const Args& a, int64_t row)
{
    const int lane = threadIdx.x & 63;
    const int NC = a.NC;
    observe();
    const double v = lane < NC ? get_f64(&a.wpart[row * NC + lane]) : 0.0;
    const double incl = wave_inclusive_scan(v);
    double* pref = a.prefw + row * (NC + 1);
    if (lane < NC) put_f64(&pref[lane + 1], incl);   // pref[NC] is the residual mass W
    if (lane == 0) {
        put_f64(&pref[0], 0.0);
        put_u32(&a.cnt2[row], 0u);
        publish();
        put_u32(&a.flag2[row], 1u);
    }
}

// ---------------------------------------------------- inverse CDF --

// Search of this block's chunk for the smallest x with
// base + sum_{chunk start <= y <= x} w(y) > T, where w is the residual
// max(0, p*Q - q*P) (RESID) or p itself.  If rounding leaves no such x in
// the chunk, the last x with w(x) > 0 is taken.  All threads must call; the
// token is returned in every thread.
template <bool RESID>
__device__ __forceinline__ int chunk_draw(const float4 (&pv)[kVec], const float4 (&qv)[kVec], double P, double Q,
                          int c, double base, double T)
{
    __shared__ double s_seg[kVec][kWaves];
    __shared__ int s_ks, s_ws;
    __shared__ double s_base;
    __shared__ int s_x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    auto wval = [&](float4 p4, float4 q4, int e) -> double {
        const double p = (double)comp(p4, e);
        if constexpr (RESID) {
            const double d = p * Q - (double)comp(q4, e) * P;
            return d > 0.0 ? d : 0.0;
        } else {
            (void)q4;
            return p;
        }
    };

    double sk[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) s += wval(pv[k], qv[k], e);
        sk[k] = s;
    }
    // segment (k, wave) = 256 consecutive values; segments in index order
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        const double s = wave_sum(sk[k]);
        if (lane == 0) s_seg[k][w] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double run = base;
        int ks = -1, ws = 0, lk = 0, lw = 0;
        double bs = base, lb = base;
        for (int k = 0; k < kVec; ++k) {
            for (int j = 0; j < kWaves; ++j) {
                const double s = s_seg[k][j];
                if (s > 0.0) {
                    lk = k;
                    lw = j;
                    lb = run;
                }
                if (ks < 0 && run + s > T) {
                    ks = k;
                    ws = j;
                    bs = run;
                }
                run += s;
            }
        }
        if (ks < 0) {               // rounding: take the last segment with mass
            ks = lk;
            ws = lw;
            bs = lb;
        }
        s_ks = ks;
        s_ws = ws;
        s_base = bs;
    }
    __syncthreads();
    const int ks = s_ks;
    if (w == s_ws) {
        float4 lp[kVec], lq[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            lp[k] = pv[k];
            lq[k] = qv[k];
        }
        reg_barrier(lp);
        reg_barrier(lq);
        // every index below is static: a uniform branch per segment row k
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            if (k != ks) continue;
            const double incl = wave_inclusive_scan(sk[k]);
            double run = __shfl_up(incl, 1);
            if (lane == 0) run = 0.0;
            run += s_base;
            int hit = -1, lastpos = -1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double v = wval(lp[k], lq[k], e);
                run += v;
                if (hit < 0 && run > T) hit = e;
                if (v > 0.0) lastpos = e;
            }
            const unsigned long long mh = __ballot(hit >= 0);
            if (mh) {
                const int l = __ffsll((unsigned long long)mh) - 1;
                if (lane == l) s_x = f4_index(c, k) * 4 + hit;
            } else {
                const unsigned long long mp = __ballot(lastpos >= 0);
                if (mp) {
                    const int l = 63 - __clzll(mp);
                    if (lane == l) s_x = f4_index(c, k) * 4 + lastpos;
                } else if (lane == 0) {
                    s_x = f4_index(c, k) * 4;   // unreachable for a segment with mass
                }
            }
        }
    }
    __syncthreads();
    return s_x;
}

// ----------------------------------------------------------- resolve --

__device__ __forceinline__ void resolve_greedy(const Args& a, int b)
{
    const int lane = threadIdx.x & 63;
    const int K = a.K;
    const int64_t r0 = (int64_t)b * (K + 1);
    observe();
    int n = K;
    for (int base = 0; base < K; base += 64) {
        const int i = base + lane;
        bool miss = false;
        if (i < K) miss = a.dt[(int64_t)b * K + i] != get_i32(&a.rowres[r0 + i].arg);
        const unsigned long long m = __ballot(miss);
        if (m) {
            n = base + __ffsll((unsigned long long)m) - 1;
            break;
        }
    }
    int next = 0;
    if (lane == 0) next = get_i32(&a.rowres[r0 + n].arg);
    next = __shfl(next, 0);   // the load has completed before any lane zeroes the row results
    if (lane == 0) {
        a.n_out[b] = n;
        a.next_out[b] = next;
        put_u32(&a.seqcnt[b], 0u);
    }
    zero_sequence_data(a, b, false);
}

__device__ __forceinline__ void resolve_sampled(const Args& a, int b)
{
    const int lane = threadIdx.x & 63;
    const int K = a.K;
    const int64_t r0 = (int64_t)b * (K + 1);
    observe();
    int n = K;
    for (int base = 0; base < K; base += 64) {
        const int i = base + lane;
        const bool rej = i < K && get_i32(&a.rowres[r0 + i].acc) == 0;
        const unsigned long long m = __ballot(rej);
        if (m) {
            n = base + __ffsll((unsigned long long)m) - 1;
            break;
        }
    }
    int next = 0;
    if (lane == 0) next = get_i32(&a.rowres[r0 + n].cand);
    next = __shfl(next, 0);   // the load has completed before any lane zeroes the row results
    if (lane == 0) {
        a.n_out[b] = n;
        a.next_out[b] = next;
        put_u32(&a.seqcnt[b], 0u);
    }
    for (int i = lane; i <= K; i += 64) {
        put_u32(&a.flag1[r0 + i], 0u);
        put_u32(&a.flag2[r0 + i], 0u);
    }
    zero_sequence_data(a, b, true);
}

// ----------------------------------------------------------- kernels --

template <bool VEC>
__global__ __launch_bounds__(kThreads) void sv_greedy_kernel(Args a)
{
    __shared__ int s_last;
    const int NC = a.NC, K = a.K;
    const unsigned per_seq = (unsigned)(K + 1) * (unsigned)NC;
    const unsigned item = blockIdx.x;
    const int b = (int)(item / per_seq);
    const unsigned r = item - (unsigned)b * per_seq;
    const int i = (int)(r / (unsigned)NC);
    const int c = (int)(r - (unsigned)i * (unsigned)NC);
    const int64_t row = (int64_t)b * (K + 1) + i;

    float4 pv[kVec];
    load_chunk<VEC>(a.tp + row * a.V, a.V, c, pv);
    const Acc t = thread_stats<false>(pv, pv, a.V, c);
    const Acc s = block_reduce<false>(t);
    if (threadIdx.x == 0) {
        ChunkPart* dst = &a.parts[row * NC + c];
        put_f64(&dst->sp, s.sp);
        put_f32(&dst->maxv, s.maxv);
        put_i32(&dst->arg, s.arg);
        publish();
        s_last = count_up(&a.cnt1[row]) == (unsigned)NC - 1u;
    }
    __syncthreads();
    if (!s_last || threadIdx.x >= 64) return;
    combine_row<false>(a, b, i, row);
    int last_row = 0;
    if (threadIdx.x == 0) {
        publish();
        last_row = count_up(&a.seqcnt[b]) == (unsigned)K;
    }
    last_row = __shfl(last_row, 0);
    if (last_row) resolve_greedy(a, b);
}

template <bool VEC>
__device__ __forceinline__ void sample_item(const Args& a, int b, int i, int c)
{
    __shared__ int s_last, s_draw, s_owner, s_resid;
    __shared__ double s_P, s_Q, s_T, s_lo;
    const int NC = a.NC, K = a.K, V = a.V;
    const int64_t row = (int64_t)b * (K + 1) + i;
    const bool pair = i < K;

    float4 pv[kVec], qv[kVec];
    load_chunk<VEC>(a.tp + row * V, V, c, pv);
    if (pair) {
        load_chunk<VEC>(a.dp + ((int64_t)b * K + i) * V, V, c, qv);
    } else {
#pragma unroll
        for (int k = 0; k < kVec; ++k) qv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const Acc t = pair ? thread_stats<true>(pv, qv, V, c) : thread_stats<false>(pv, qv, V, c);
    reg_barrier(pv);
    reg_barrier(qv);
    const Acc s = pair ? block_reduce<true>(t) : block_reduce<false>(t);

    // rendezvous 1: row masses, argmax, acceptance
    if (threadIdx.x == 0) {
        ChunkPart* dst = &a.parts[row * NC + c];
        put_f64(&dst->sp, s.sp);
        if (pair) {
            put_f64(&dst->sq, s.sq);
            put_f64(&dst->smin, s.smin);
        }
        put_f32(&dst->maxv, s.maxv);
        put_i32(&dst->arg, s.arg);
        publish();
        s_last = count_up(&a.cnt1[row]) == (unsigned)NC - 1u;
    }
    __syncthreads();
    if (s_last) {
        if (threadIdx.x < 64) combine_row<true>(a, b, i, row);
    } else if (threadIdx.x == 0) {
        wait_flag(&a.flag1[row], a.hdr, a.wait_ticks);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const RowRes* rr = &a.rowres[row];
        s_P = get_f64(&rr->P);
        s_Q = get_f64(&rr->Q);
        s_draw = get_i32(&rr->draw);
    }
    __syncthreads();
    const double P = s_P, Q = s_Q;

    if (s_draw) {
        const double uK = (double)a.u[(int64_t)b * (K + 1) + K];
        if (pair) {
            // rendezvous 2: residual masses of the rejecting row
            double wsum = 0.0;
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double d = (double)comp(pv[k], e) * Q - (double)comp(qv[k], e) * P;
                    wsum += d > 0.0 ? d : 0.0;
                }
            }
            wsum = block_sum(wsum);
            if (threadIdx.x == 0) {
                put_f64(&a.wpart[row * NC + c], wsum);
                publish();
                s_last = count_up(&a.cnt2[row]) == (unsigned)NC - 1u;
            }
            __syncthreads();
            if (s_last) {
                if (threadIdx.x < 64) combine_residual(a, row);
            } else if (threadIdx.x == 0) {
                wait_flag(&a.flag2[row], a.hdr, a.wait_ticks);
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            const double* pref = a.prefp + row * (NC + 1);
            double mass = P;
            int resid = 0;
            if (pair) {
                const double W = get_f64(&a.prefw[row * (NC + 1) + NC]);
                if (W > 0.0) {
                    pref = a.prefw + row * (NC + 1);
                    mass = W;
                    resid = 1;
                }
            }
            const double T = uK * mass;
            const double lo = get_f64(&pref[c]), hi = get_f64(&pref[c + 1]);
            s_owner = (lo <= T && T < hi) ? 1 : 0;
            s_resid = resid;
            s_T = T;
            s_lo = lo;
        }
        __syncthreads();
        if (s_owner) {
            const int x = s_resid ? chunk_draw<true>(pv, qv, P, Q, c, s_lo, s_T)
                                  : chunk_draw<false>(pv, qv, P, Q, c, s_lo, s_T);
            if (threadIdx.x == 0) put_i32(&a.rowres[row].cand, x);
        }
    }

    // sequence completion
    if (threadIdx.x == 0) {
        const unsigned per_seq = (unsigned)(K + 1) * (unsigned)NC;
        publish();
        s_last = count_up(&a.seqcnt[b]) == per_seq - 1u;
    }
    __syncthreads();
    if (s_last && threadIdx.x < 64) resolve_sampled(a, b);
    __syncthreads();
}

template <bool VEC>
__global__ __launch_bounds__(kThreads, 2) void sv_sample_kernel(Args a)
{
    __shared__ unsigned s_ticket;
    const unsigned per_seq = (unsigned)(a.K + 1) * (unsigned)a.NC;
    for (;;) {
        if (threadIdx.x == 0) s_ticket = count_up(&a.hdr->ticket);   // carries no data
        __syncthreads();
        const unsigned tk = s_ticket;
        __syncthreads();
        if (tk >= a.total) break;
        const int b = (int)(tk / per_seq);
        const unsigned r = tk - (unsigned)b * per_seq;
        const int i = (int)(r / (unsigned)a.NC);
        const int c = (int)(r - (unsigned)i * (unsigned)a.NC);
        sample_item<VEC>(a, b, i, c);
    }
    if (threadIdx.x == 0) {
        if (count_up(&a.hdr->exit_count) == gridDim.x - 1u) {
            put_u32(&a.hdr->ticket, 0u);     // every block has taken its last ticket
            put_u32(&a.hdr->exit_count, 0u);
        }
    }
}

__global__ void sv_fill_zero_kernel(uint4* p, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n16; j += stride)
        p[j] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------- host --

struct DevInfo {
    int cus = 0;
    int wall_khz = 0;
    int occ[2] = {0, 0};     // resident sampled blocks per CU: scalar, vector path
    bool ok = false;
};

std::mutex g_mu;
DevInfo g_dev[64];

sv_status device_info(DevInfo* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DevInfo& d = g_dev[dev];
    if (!d.ok) {
        int cus = 0, o0 = 0, o1 = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return SV_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o0, sv_sample_kernel<false>, kThreads, 0) != hipSuccess)
            return SV_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o1, sv_sample_kernel<true>, kThreads, 0) != hipSuccess)
            return SV_ERR_HIP;
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
            khz = 100000;   // gfx9 wall clock: 100 MHz
        d.wall_khz = khz;
        d.cus = cus;
        d.occ[0] = o0;
        d.occ[1] = o1;
        d.ok = true;
    }
    *out = d;
    return SV_OK;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

sv_status check_sizes(int32_t B, int32_t K, int32_t V)
{
    if (B < 0 || K < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (V > SV_MAX_V || K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
    const uint64_t NC = ((uint64_t)V + kChunk - 1) / kChunk;
    if ((uint64_t)B * (uint64_t)(K + 1) * NC >= (1ull << 31)) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

Args make_args(void* ws, int32_t B, int32_t K, int32_t V)
{
    Args a{};
    const int NC = (V + kChunk - 1) / kChunk;
    const Layout L = make_layout(B, K, NC);
    unsigned char* w = static_cast<unsigned char*>(ws);
    a.hdr = reinterpret_cast<Header*>(w + L.hdr);
    a.cnt1 = reinterpret_cast<unsigned*>(w + L.cnt1);
    a.cnt2 = reinterpret_cast<unsigned*>(w + L.cnt2);
    a.flag1 = reinterpret_cast<unsigned*>(w + L.flag1);
    a.flag2 = reinterpret_cast<unsigned*>(w + L.flag2);
    a.seqcnt = reinterpret_cast<unsigned*>(w + L.seqcnt);
    a.rowres = reinterpret_cast<RowRes*>(w + L.rowres);
    a.parts = reinterpret_cast<ChunkPart*>(w + L.parts);
    a.wpart = reinterpret_cast<double*>(w + L.wpart);
    a.prefp = reinterpret_cast<double*>(w + L.prefp);
    a.prefw = reinterpret_cast<double*>(w + L.prefw);
    a.B = B;
    a.K = K;
    a.V = V;
    a.NC = NC;
    a.total = (unsigned)((uint64_t)B * (uint64_t)(K + 1) * (uint64_t)NC);
    return a;
}

}  // namespace

extern "C" {

size_t sv_workspace_size(int32_t B, int32_t K, int32_t V, int32_t sampled)
{
    (void)sampled;   // both modes share one layout
    if (check_sizes(B, K, V) != SV_OK) return 0;
    const int NC = (V + kChunk - 1) / kChunk;
    return make_layout(B, K, NC).total;
}

sv_status sv_workspace_init(void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || !aligned(workspace, 16)) return SV_ERR_WORKSPACE;
    const size_t n16 = workspace_bytes / 16;
    if (n16 == 0) return SV_OK;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(sv_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint4*>(workspace), n16);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_verify_greedy_batched(const float* target_probs, const int32_t* draft_tokens,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t* n_accepted, int32_t* next_token,
                                   void* workspace, size_t workspace_bytes,
                                   sv_row_stats* stats, void* stream)
{
    sv_status st = check_sizes(B, K, V);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;   // nothing to verify; pointers are not inspected
    if (!target_probs || !n_accepted || !next_token || (K > 0 && !draft_tokens))
        return SV_ERR_INVALID_ARG;
    if (!aligned(target_probs, 4) || !aligned(draft_tokens, 4) || !aligned(n_accepted, 4) ||
        !aligned(next_token, 4) || !aligned(stats, 8))
        return SV_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < sv_workspace_size(B, K, V, 0))
        return SV_ERR_WORKSPACE;
    Args a = make_args(workspace, B, K, V);
    a.tp = target_probs;
    a.dt = draft_tokens;
    a.n_out = n_accepted;
    a.next_out = next_token;
    a.stats = stats;
    const bool vec = (V % 4 == 0) && aligned(target_probs, 16);
    const dim3 grid(a.total), block(kThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vec)
        hipLaunchKernelGGL(sv_greedy_kernel<true>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(sv_greedy_kernel<false>, grid, block, 0, s, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_verify_sample_batched(const float* target_probs, const float* draft_probs,
                                   const int32_t* draft_tokens, const float* uniforms,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t* n_accepted, int32_t* next_token,
                                   void* workspace, size_t workspace_bytes,
                                   sv_row_stats* stats, void* stream)
{
    sv_status st = check_sizes(B, K, V);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;   // nothing to verify; pointers are not inspected
    if (!target_probs || !uniforms || !n_accepted || !next_token ||
        (K > 0 && (!draft_probs || !draft_tokens)))
        return SV_ERR_INVALID_ARG;
    if (!aligned(target_probs, 4) || !aligned(draft_probs, 4) || !aligned(draft_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(n_accepted, 4) || !aligned(next_token, 4) ||
        !aligned(stats, 8))
        return SV_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < sv_workspace_size(B, K, V, 1))
        return SV_ERR_WORKSPACE;
    DevInfo d;
    st = device_info(&d);
    if (st != SV_OK) return st;
    Args a = make_args(workspace, B, K, V);
    a.tp = target_probs;
    a.dp = draft_probs;
    a.dt = draft_tokens;
    a.u = uniforms;
    a.n_out = n_accepted;
    a.next_out = next_token;
    a.stats = stats;
    a.wait_ticks = (unsigned long long)(kWaitSeconds * 1000.0 * (double)d.wall_khz);
    const bool vec = (V % 4 == 0) && aligned(target_probs, 16) && aligned(draft_probs, 16);
    const int occ = d.occ[vec ? 1 : 0];
    const uint64_t resident = (uint64_t)occ * (uint64_t)d.cus;
    // the row rendezvous needs every chunk of one row resident at once
    if (resident < (uint64_t)a.NC) return SV_ERR_UNSUPPORTED;
    const unsigned grid = (unsigned)(resident < a.total ? resident : a.total);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vec)
        hipLaunchKernelGGL(sv_sample_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(sv_sample_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_workspace_error(const void* workspace, int32_t* error_out, void* stream)
{
    if (!workspace || !error_out) return SV_ERR_INVALID_ARG;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SV_ERR_HIP;
    unsigned v = 0;
    const unsigned char* w = static_cast<const unsigned char*>(workspace);
    if (hipMemcpy(&v, w + offsetof(Header, error), sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return SV_ERR_HIP;
    *error_out = (int32_t)v;
    return SV_OK;
}

const char* sv_status_string(sv_status s)
{
    switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG: NULL, misaligned or negative argument";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SV_ERR_HIP: return "SV_ERR_HIP: a HIP runtime call or kernel launch failed";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: size beyond the supported maximum";
    }
    return "unknown sv_status";
}

}  // extern "C"
