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
//     256-thread block (4 waves) streams one chunk of one row (and, in
//     sampled mode, the same chunk of the matching draft row): each thread
//     issues 8 coalesced, non-temporal 16-byte loads per operand;
//   * per-chunk partials (fp64 masses, lowest-index argmax) are combined in
//     lane (= chunk) order by the last block of the row to arrive, so every
//     result depends on V alone, never on B, K, the launch shape or timing;
//   * the last row of a sequence to complete resolves the accept-prefix
//     length n (the first rejected draft, or K);
//   * greedy: next token = argmax of row n; no block ever waits.
//   * sampled: a persistent grid takes work tickets in order.  Row tickets
//     (pass 1) never wait.  For each sequence b, NC residual tickets follow
//     kLag sequences later in the ticket order; by then b is normally
//     resolved and its rows were streamed moments ago, so the residual
//     re-read of the rejected pair (p_n, q_n) is served by the Infinity Cache
//     rather than HBM.  Each residual ticket adds its chunk's mass of
//     w = max(0, p_n*Q - q_n*P); the last one combines them and the block
//     whose chunk holds u_K * W runs the inverse-CDF search over that chunk.
//     When every draft is accepted, the resolver draws the bonus token from
//     p_K the same way (chunk masses of p_K locate the chunk), and the
//     sequence's residual tickets do nothing but count.
//
// Progress: the only wait is a residual ticket whose sequence is not yet
// resolved.  All of that sequence's row tickets come earlier in the ticket
// order, so they are held by running blocks, and row tickets never wait:
// the sequence resolves.  The wait is also bounded in time (expiry raises
// the workspace fault word instead of spinning forever).

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
constexpr int kLag = 16;                       // residual tickets trail their sequence
constexpr unsigned kTicketBatch = 4;           // tickets per atomic on large launches
constexpr double kWaitSeconds = 2.0;           // bound of the one cross-block wait

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

struct RowRes {              // 32 bytes
    double P, Q;             // row masses
    int acc, arg;            // acceptance bit of the row's draft, lowest-index argmax
    int pad[2];
};

struct SeqInfo {             // 8 bytes
    int n;                   // accept-prefix length
    unsigned resolved;       // 1 once n is published
};

struct Layout {
    size_t hdr, cnt1, cnt2, seqcnt, seqinfo, rowres, parts, wpart, zero, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline Layout make_layout(int64_t B, int64_t K, int64_t NC)
{
    const size_t R = (size_t)(B * (K + 1));
    Layout L{};
    size_t o = 0;
    L.hdr = o;     o = align_up(o + sizeof(Header), 256);
    L.cnt1 = o;    o = align_up(o + R * 4, 256);
    L.cnt2 = o;    o = align_up(o + (size_t)B * 4, 256);
    L.seqcnt = o;  o = align_up(o + (size_t)B * 4, 256);
    L.seqinfo = o; o = align_up(o + (size_t)B * sizeof(SeqInfo), 256);
    L.rowres = o;  o = align_up(o + R * sizeof(RowRes), 256);
    L.parts = o;   o = align_up(o + R * (size_t)NC * sizeof(ChunkPart), 256);
    L.wpart = o;   o = align_up(o + (size_t)B * (size_t)NC * 8, 256);
    L.zero = o;    o = align_up(o + (size_t)kChunk * 4, 256);   // never written
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
    unsigned *cnt1, *cnt2, *seqcnt;
    SeqInfo* seqinfo;
    RowRes* rowres;
    ChunkPart* parts;
    double* wpart;
    const float* zero;       // one chunk of zeros (the bonus row's draft operand)
    int B, K, V, NC;
    int lag;                 // min(kLag, B)
    unsigned batch;          // tickets per atomic (sampled)
    unsigned total;          // work tickets (sampled)
    unsigned long long wait_ticks;   // wait bound in wall-clock ticks
};

// ------------------------------------------- cross-block communication --
//
// Every value one block publishes for another (chunk partials, row results,
// counters) is written and read with agent-scope atomic accesses.  On gfx950
// these are performed at the device-coherent level (sc1 loads and stores;
// RMW atomics at the memory side) instead of in the per-XCD L2, so no L2
// write-back or invalidate (the cost of agent-scope release/acquire fences)
// is ever needed.  Ordering is explicit:
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

// Bounded wait until *flag != 0; on expiry raises the fault word and returns
// (the call's outputs are then unspecified, but every block exits).
__device__ __forceinline__ void wait_flag(const unsigned* flag, Header* hdr, unsigned long long ticks)
{
    const unsigned long long t0 = wall_clock64();
    while (get_u32(flag) == 0u) {
        __builtin_amdgcn_s_sleep(8);
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

// Once sequence b is finished nothing reads its counters, partials or row
// results again: return them to zero so that the whole workspace is zero
// between calls, whatever shapes the next call uses.  One wave calls it.
__device__ __forceinline__ void zero_sequence(const Args& a, int b)
{
    const int64_t rows = a.K + 1, r0 = (int64_t)b * rows, NC = a.NC;
    wave_zero(a.parts + r0 * NC, (size_t)(rows * NC) * sizeof(ChunkPart));
    wave_zero(a.rowres + r0, (size_t)rows * sizeof(RowRes));
    wave_zero(a.wpart + (int64_t)b * NC, (size_t)NC * 8);
    for (int64_t j = threadIdx.x & 63; j < rows; j += 64) put_u32(&a.cnt1[r0 + j], 0u);
    if ((threadIdx.x & 63) == 0) {
        put_u32(&a.cnt2[b], 0u);
        put_u32(&a.seqcnt[b], 0u);
        put_u64(&a.seqinfo[b], 0ull);
    }
}

// ---------------------------------------------------------- chunk I/O --

// Thread t holds float4 number (c * kChunk4 + k * 256 + t) of the row, k < 8:
// consecutive threads read consecutive 16-byte words (fully coalesced).
__device__ __forceinline__ int f4_index(int c, int k) { return c * kChunk4 + k * kThreads + (int)threadIdx.x; }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming load: every value is read once, so it is not kept in cache.
__device__ __forceinline__ float4 load_stream(const float4* p)
{
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float load_stream(const float* p) { return __builtin_nontemporal_load(p); }

// Loads of float4 numbers k in [0, kVec) of chunk c.  Every load is
// unconditional (an out-of-range index is clamped to the row's last element)
// and nothing is written to the destination registers afterwards: values
// past the row's end are masked where they are consumed (thread_stats), so
// all loads of a thread are in flight together.  STREAM selects the
// non-temporal hint (first pass) or ordinary cached loads.
template <bool VEC, bool STREAM>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int V, int c, float4 (&v)[kVec])
{
    if constexpr (VEC) {
        const float4* r4 = reinterpret_cast<const float4*>(row);
        const int nf = V >> 2;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const int f = f4_index(c, k);
            const float4* src = r4 + (f < nf ? f : nf - 1);
            v[k] = STREAM ? load_stream(src) : *src;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const int x = f4_index(c, k) * 4;
            float e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float* src = row + (x + j < V ? x + j : V - 1);
                e[j] = STREAM ? load_stream(src) : *src;
            }
            v[k] = make_float4(e[0], e[1], e[2], e[3]);
        }
    }
}

// Cached load of float4 number k (runtime) of chunk c, zero outside the row.
template <bool VEC>
__device__ __forceinline__ float4 load_one(const float* __restrict__ row, int V, int c, int k)
{
    if constexpr (VEC) {
        const float4* r4 = reinterpret_cast<const float4*>(row);
        const int nf = V >> 2, f = f4_index(c, k);
        const float4 v = r4[f < nf ? f : nf - 1];
        return f < nf ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        const int x = f4_index(c, k) * 4;
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = row[x + j < V ? x + j : V - 1];
        return make_float4(x + 0 < V ? e[0] : 0.f, x + 1 < V ? e[1] : 0.f,
                           x + 2 < V ? e[2] : 0.f, x + 3 < V ? e[3] : 0.f);
    }
}

__device__ __forceinline__ float comp(float4 v, int e)
{
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// Residual mass of one value: max(0, p*Q - q*P), fp64, no contraction.
__device__ __forceinline__ double resid(float p, float q, double P, double Q)
{
    const double d = (double)p * Q - (double)q * P;
    return d > 0.0 ? d : 0.0;
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

// Per-thread partials of one chunk as load_chunk left it: values at index
// V or beyond (clamped duplicates) are masked to 0 here.
template <bool PAIR>
__device__ __forceinline__ Acc thread_stats(const float4 (&pv)[kVec], const float4 (&qv)[kVec], int V, int c)
{
    Acc a{0.0, 0.0, 0.0, -INFINITY, INT_MAX};
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        const int x0 = f4_index(c, k) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = x0 + e < V;
            const float p = in ? comp(pv[k], e) : 0.0f;
            if (in && p > a.maxv) {
                a.maxv = p;
                a.arg = x0 + e;
            }
            a.sp += (double)p;
            if constexpr (PAIR) {
                const float q = in ? comp(qv[k], e) : 0.0f;
                a.sq += (double)q;
                a.smin += (double)fminf(p, q);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep fp64 temporaries to one float4 at a time
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

struct RowView {
    double P, Q, Smin;       // row masses
    float maxv;
    int arg;
};

// Wave-cooperative (all 64 lanes of one wave): combine the NC chunk partials
// of a row in lane (= chunk) order.
template <bool PAIR>
__device__ __forceinline__ RowView combine_row(const ChunkPart* parts, int NC)
{
    const int lane = threadIdx.x & 63;
    observe();
    double sp = 0.0, sq = 0.0, sm = 0.0;
    float mv = -INFINITY;
    int ai = INT_MAX;
    if (lane < NC) {
        sp = get_f64(&parts[lane].sp);
        if constexpr (PAIR) {
            sq = get_f64(&parts[lane].sq);
            sm = get_f64(&parts[lane].smin);
        }
        mv = get_f32(&parts[lane].maxv);
        ai = get_i32(&parts[lane].arg);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(mv, off);
        const int oi = __shfl_xor(ai, off);
        argmax_merge(mv, ai, ov, oi);
    }
    const double incl = wave_inclusive_scan(sp);
    RowView r;
    r.P = __shfl(incl, NC - 1);
    r.Q = PAIR ? wave_sum(sq) : 0.0;
    r.Smin = PAIR ? wave_sum(sm) : 0.0;
    r.maxv = mv;
    r.arg = ai;
    return r;
}

// Wave-cooperative: given the NC chunk masses m[c] (lane c), the chunk that
// holds T = u * (total) -- the one with prefix(c-1) <= T < prefix(c) -- and
// its base prefix(c-1).  Prefixes are the inclusive scan in lane order; the
// total is its last entry, so T < total always has an owner when total > 0.
// Returns the total; *owner = -1 when no chunk qualifies (total == 0).
__device__ __forceinline__ double locate_chunk(double m, int NC, double u, int* owner, double* base,
                                               double* T_out)
{
    const int lane = threadIdx.x & 63;
    const double incl = wave_inclusive_scan(lane < NC ? m : 0.0);
    const double total = __shfl(incl, NC - 1);
    const double T = u * total;
    double lo = __shfl_up(incl, 1);
    if (lane == 0) lo = 0.0;
    const bool own = lane < NC && lo <= T && T < incl;
    const unsigned long long mk = __ballot(own);
    const int c = mk ? __ffsll((unsigned long long)mk) - 1 : -1;
    *owner = c;
    *base = c >= 0 ? __shfl(lo, c) : 0.0;
    *T_out = T;
    return total;
}

// ---------------------------------------------------- inverse CDF --

// Search of chunk c for the smallest x with
// base + sum_{chunk start <= y <= x} w(y) > T, where w is the residual
// max(0, p*Q - q*P) (RESID) or p itself.  If rounding leaves no such x in
// the chunk, the last x with w(x) > 0 is taken.  The chunk is re-read with
// cached loads a few float4s per thread at a time, and the selected segment
// once more for the final scan (few registers; a rare path).  All threads of
// the block must call; the token is returned in every thread.
template <bool VEC, bool RESID>
__device__ __noinline__ int chunk_draw(const float* prow, const float* qrow, int V, double P, double Q,
                                       int c, double base, double T)
{
    __shared__ double s_seg[kVec][kWaves];
    __shared__ int s_ks, s_ws;
    __shared__ double s_base;
    __shared__ int s_x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    auto wsum4 = [&](float4 p4, float4 q4) -> double {   // one float4, in index order
        double t = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            t += RESID ? resid(comp(p4, e), comp(q4, e), P, Q) : (double)comp(p4, e);
        return t;
    };

    // segment (k, wave) = 256 consecutive values; segments in index order
#pragma unroll 4
    for (int k = 0; k < kVec; ++k) {
        const float4 p4 = load_one<VEC>(prow, V, c, k);
        const float4 q4 = RESID ? load_one<VEC>(qrow, V, c, k) : p4;
        const double s = wave_sum(wsum4(p4, q4));
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
    if (w == s_ws) {
        const int k = s_ks;
        const float4 p4 = load_one<VEC>(prow, V, c, k);
        const float4 q4 = RESID ? load_one<VEC>(qrow, V, c, k) : p4;
        const double incl = wave_inclusive_scan(wsum4(p4, q4));
        double run = __shfl_up(incl, 1);
        if (lane == 0) run = 0.0;
        run += s_base;
        int hit = -1, lastpos = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double v = RESID ? resid(comp(p4, e), comp(q4, e), P, Q) : (double)comp(p4, e);
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
    __syncthreads();
    return s_x;
}

__device__ __forceinline__ void write_stats(const Args& a, int64_t row, const RowView& rv, bool pair,
                                            float pt, float qt, bool has_t)
{
    sv_row_stats s;
    s.argmax = rv.arg;
    s.max_p = rv.maxv;
    s.sum_p = rv.P;
    s.sum_q = pair ? rv.Q : 0.0;
    s.sum_min = pair ? rv.Smin : 0.0;
    s.sum_pos = pair ? rv.P - rv.Smin : 0.0;
    s.p_t = has_t ? pt : 0.0f;
    s.q_t = pair ? qt : 0.0f;
    a.stats[row] = s;
}

// Wave-cooperative: the accept-prefix length of sequence b from the rows'
// published acceptance bits.
__device__ __forceinline__ int first_rejection(const Args& a, int b)
{
    const int lane = threadIdx.x & 63, K = a.K;
    const int64_t r0 = (int64_t)b * (K + 1);
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
    return n;
}

// ----------------------------------------------------------- greedy --

template <bool VEC>
__global__ __launch_bounds__(kThreads) void sv_greedy_kernel(Args a)
{
    __shared__ int s_last;
    const int NC = a.NC, K = a.K, V = a.V;
    const unsigned per_seq = (unsigned)(K + 1) * (unsigned)NC;
    const unsigned item = blockIdx.x;
    const int b = (int)(item / per_seq);
    const unsigned r = item - (unsigned)b * per_seq;
    const int i = (int)(r / (unsigned)NC);
    const int c = (int)(r - (unsigned)i * (unsigned)NC);
    const int64_t row = (int64_t)b * (K + 1) + i;

    float4 pv[kVec];
    load_chunk<VEC, true>(a.tp + row * V, V, c, pv);
    const Acc t = thread_stats<false>(pv, pv, V, c);
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
    // wave 0 of the last block of the row
    const RowView rv = combine_row<false>(a.parts + row * NC, NC);
    int last_row = 0;
    if (threadIdx.x == 0) {
        put_i32(&a.rowres[row].arg, rv.arg);
        if (a.stats) {
            const int tk = i < K ? a.dt[(int64_t)b * K + i] : -1;
            const bool tin = tk >= 0 && tk < V;
            write_stats(a, row, rv, false, tin ? a.tp[row * V + tk] : 0.0f, 0.0f, i < K);
        }
        publish();
        last_row = count_up(&a.seqcnt[b]) == (unsigned)K;
    }
    last_row = __shfl(last_row, 0);
    if (!last_row) return;
    // the sequence's last row: n = first draft that differs from its argmax
    observe();
    const int64_t r0 = (int64_t)b * (K + 1);
    const int lane = threadIdx.x;
    int n = K;
    for (int base = 0; base < K; base += 64) {
        const int j = base + lane;
        const bool miss = j < K && a.dt[(int64_t)b * K + j] != get_i32(&a.rowres[r0 + j].arg);
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
    }
    zero_sequence(a, b);
}

// ---------------------------------------------------------- sampled --

// Row ticket: chunk c of target row i of sequence b, with the same chunk of
// draft row i (the zero chunk for the bonus row i == K, so that both kinds
// run the same straight-line loads).
template <bool VEC>
__device__ __forceinline__ void row_item(const Args& a, int b, int i, int c)
{
    __shared__ int s_last, s_n, s_owner;
    __shared__ double s_base, s_T, s_P;
    const int NC = a.NC, K = a.K, V = a.V;
    const int64_t row = (int64_t)b * (K + 1) + i;
    const bool pair = i < K;
    const float* prow = a.tp + row * V;
    const float* qrow = pair ? a.dp + ((int64_t)b * K + i) * V : a.zero;
    const int qV = pair ? V : kChunk;       // the zero operand is one chunk long
    const int qc = pair ? c : 0;

    float4 pv[kVec], qv[kVec];
    load_chunk<VEC, true>(prow, V, c, pv);
    load_chunk<VEC, true>(qrow, qV, qc, qv);
    const Acc t = thread_stats<true>(pv, qv, V, c);
    const Acc s = block_reduce<true>(t);

    if (threadIdx.x == 0) {
        ChunkPart* dst = &a.parts[row * NC + c];
        put_f64(&dst->sp, s.sp);
        put_f64(&dst->sq, s.sq);
        put_f64(&dst->smin, s.smin);
        put_f32(&dst->maxv, s.maxv);
        put_i32(&dst->arg, s.arg);
        publish();
        s_last = count_up(&a.cnt1[row]) == (unsigned)NC - 1u;
    }
    __syncthreads();
    if (!s_last) return;

    // last block of the row: combine it, decide its draft's acceptance
    if (threadIdx.x < 64) {
        const RowView rv = combine_row<true>(a.parts + row * NC, NC);
        int last_row = 0;
        if (threadIdx.x == 0) {
            const int tk = pair ? a.dt[(int64_t)b * K + i] : -1;
            const bool tin = tk >= 0 && tk < V;
            const float pt = tin ? prow[tk] : 0.0f;
            const float qt = tin ? qrow[tk] : 0.0f;
            int acc = 1;
            if (pair) {
                const double ui = (double)a.u[(int64_t)b * (K + 1) + i];
                acc = (ui * (double)qt * rv.P < (double)pt * rv.Q) ? 1 : 0;
            }
            RowRes* rr = &a.rowres[row];
            put_f64(&rr->P, rv.P);
            put_f64(&rr->Q, rv.Q);
            put_i32(&rr->acc, acc);
            put_i32(&rr->arg, rv.arg);
            if (a.stats) write_stats(a, row, rv, pair, pt, qt, pair);
            publish();
            last_row = count_up(&a.seqcnt[b]) == (unsigned)K;
        }
        last_row = __shfl(last_row, 0);
        int n = -1;
        if (last_row) {
            // the sequence's last row: accept-prefix length, and the bonus
            // chunk when every draft was accepted
            observe();
            n = first_rejection(a, b);
            if (n == K) {
                const int64_t rk = (int64_t)b * (K + 1) + K;
                const double m = threadIdx.x < NC ? get_f64(&a.parts[rk * NC + threadIdx.x].sp) : 0.0;
                int owner;
                double base, T;
                const double uK = (double)a.u[(int64_t)b * (K + 1) + K];
                const double P = locate_chunk(m, NC, uK, &owner, &base, &T);
                if (threadIdx.x == 0) {
                    s_owner = owner;
                    s_base = base;
                    s_T = T;
                    s_P = P;
                }
            }
        }
        if (threadIdx.x == 0) s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    if (n < 0) return;                       // not the sequence's last row
    if (n < K) {
        // the residual tickets of this sequence take over
        if (threadIdx.x == 0) {
            put_i32(&a.seqinfo[b].n, n);
            publish();
            put_u32(&a.seqinfo[b].resolved, 1u);
        }
        return;
    }
    // every draft accepted: draw the bonus token from p_K
    const int64_t rk = (int64_t)b * (K + 1) + K;
    int x = -1;
    if (s_owner >= 0) x = chunk_draw<VEC, false>(a.tp + rk * V, a.tp + rk * V, V, s_P, 0.0, s_owner, s_base, s_T);
    if (threadIdx.x == 0) {
        a.n_out[b] = K;
        a.next_out[b] = x;
        put_i32(&a.seqinfo[b].n, K);
        publish();
        put_u32(&a.seqinfo[b].resolved, 1u);
    }
}

// Residual ticket: chunk c of the residual row of sequence b.
template <bool VEC>
__device__ __forceinline__ void resid_item(const Args& a, int b, int c)
{
    __shared__ int s_n, s_last, s_owner, s_resid;
    __shared__ double s_P, s_Q, s_base, s_T;
    const int NC = a.NC, K = a.K, V = a.V;
    if (threadIdx.x == 0) {
        wait_flag(&a.seqinfo[b].resolved, a.hdr, a.wait_ticks);
        const int n = get_i32(&a.seqinfo[b].n);
        s_n = n;
        if (n < K) {
            const RowRes* rr = &a.rowres[(int64_t)b * (K + 1) + n];
            s_P = get_f64(&rr->P);
            s_Q = get_f64(&rr->Q);
        }
    }
    __syncthreads();
    const int n = s_n;
    if (n >= K) {                            // nothing to draw: count, and clean up last
        if (threadIdx.x == 0) s_last = count_up(&a.cnt2[b]) == (unsigned)NC - 1u;
        __syncthreads();
        if (s_last && threadIdx.x < 64) {
            observe();
            zero_sequence(a, b);
        }
        return;
    }
    const int64_t row = (int64_t)b * (K + 1) + n;
    const float* prow = a.tp + row * V;
    const float* qrow = a.dp + ((int64_t)b * K + n) * V;
    const double P = s_P, Q = s_Q;

    // this chunk's residual mass (the rows were streamed moments ago, so
    // these cached loads hit the Infinity Cache); a quarter chunk at a time
    double w = 0.0;
#pragma unroll 4
    for (int k = 0; k < kVec; ++k) {
        const float4 p4 = load_one<VEC>(prow, V, c, k), q4 = load_one<VEC>(qrow, V, c, k);
#pragma unroll
        for (int e = 0; e < 4; ++e) w += resid(comp(p4, e), comp(q4, e), P, Q);
    }
    w = block_sum(w);
    if (threadIdx.x == 0) {
        put_f64(&a.wpart[(int64_t)b * NC + c], w);
        publish();
        s_last = count_up(&a.cnt2[b]) == (unsigned)NC - 1u;
    }
    __syncthreads();
    if (!s_last) return;

    // last residual ticket: locate the chunk of u_K * W and draw there
    if (threadIdx.x < 64) {
        observe();
        const double uK = (double)a.u[(int64_t)b * (K + 1) + K];
        const double m = threadIdx.x < NC ? get_f64(&a.wpart[(int64_t)b * NC + threadIdx.x]) : 0.0;
        int owner;
        double base, T;
        const double W = locate_chunk(m, NC, uK, &owner, &base, &T);
        int rs = 1;
        if (!(W > 0.0)) {
            // rounding left no residual mass: draw from p_n itself
            const double mp = threadIdx.x < NC ? get_f64(&a.parts[row * NC + threadIdx.x].sp) : 0.0;
            locate_chunk(mp, NC, uK, &owner, &base, &T);
            rs = 0;
        }
        if (threadIdx.x == 0) {
            s_owner = owner;
            s_base = base;
            s_T = T;
            s_resid = rs;
        }
    }
    __syncthreads();
    int x = -1;
    if (s_owner >= 0)
        x = s_resid ? chunk_draw<VEC, true>(prow, qrow, V, P, Q, s_owner, s_base, s_T)
                    : chunk_draw<VEC, false>(prow, prow, V, P, Q, s_owner, s_base, s_T);
    if (threadIdx.x < 64) {
        if (threadIdx.x == 0) {
            a.n_out[b] = n;
            a.next_out[b] = x;
        }
        zero_sequence(a, b);
    }
}

// Ticket order: sequences in order; row tickets of sequence r are followed
// by the residual tickets of sequence r - lag.
struct Ticket {
    int kind;                // 0 row, 1 residual
    int b, i, c;
};

__device__ __forceinline__ Ticket decode(const Args& a, unsigned tk)
{
    const unsigned NC = (unsigned)a.NC, P1 = (unsigned)(a.K + 1) * NC, RI = NC;
    const unsigned D = (unsigned)a.lag, Bs = (unsigned)a.B;
    const unsigned partA = D * P1, partB = (Bs - D) * (P1 + RI);
    Ticket t{};
    if (tk < partA) {
        const unsigned r = tk / P1, off = tk - r * P1;
        t = Ticket{0, (int)r, (int)(off / NC), (int)(off % NC)};
    } else if (tk < partA + partB) {
        const unsigned x = tk - partA, r = D + x / (P1 + RI), off = x % (P1 + RI);
        if (off < P1)
            t = Ticket{0, (int)r, (int)(off / NC), (int)(off % NC)};
        else
            t = Ticket{1, (int)(r - D), 0, (int)(off - P1)};
    } else {
        const unsigned x = tk - partA - partB;
        t = Ticket{1, (int)(Bs - D + x / RI), 0, (int)(x % RI)};
    }
    return t;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads, 4) void sv_sample_kernel(Args a)
{
    __shared__ unsigned s_ticket;
    for (;;) {
        // one atomic hands out kTicketBatch consecutive tickets: the counter
        // is the one hot address of the launch.  A block processes its batch
        // in order; the progress argument holds because a block waits only on
        // a sequence whose row tickets all precede its current ticket.
        if (threadIdx.x == 0) s_ticket = a.batch * count_up(&a.hdr->ticket);
        __syncthreads();
        const unsigned tk0 = __builtin_amdgcn_readfirstlane(s_ticket);
        __syncthreads();
        if (tk0 >= a.total) break;
        for (unsigned tk = tk0; tk < tk0 + a.batch && tk < a.total; ++tk) {
            const Ticket t = decode(a, tk);
            if (t.kind == 0)
                row_item<VEC>(a, t.b, t.i, t.c);
            else
                resid_item<VEC>(a, t.b, t.c);
            __syncthreads();
        }
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
    if ((uint64_t)B * (uint64_t)(K + 2) * NC >= (1ull << 31)) return SV_ERR_UNSUPPORTED;
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
    a.seqcnt = reinterpret_cast<unsigned*>(w + L.seqcnt);
    a.seqinfo = reinterpret_cast<SeqInfo*>(w + L.seqinfo);
    a.rowres = reinterpret_cast<RowRes*>(w + L.rowres);
    a.parts = reinterpret_cast<ChunkPart*>(w + L.parts);
    a.wpart = reinterpret_cast<double*>(w + L.wpart);
    a.zero = reinterpret_cast<const float*>(w + L.zero);
    a.B = B;
    a.K = K;
    a.V = V;
    a.NC = NC;
    a.lag = B < kLag ? B : kLag;
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
    a.total = (unsigned)((uint64_t)B * (uint64_t)(K + 1) * (uint64_t)a.NC);
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
    a.total = (unsigned)((uint64_t)B * (uint64_t)(K + 2) * (uint64_t)a.NC);   // row + residual tickets
    const bool vec = (V % 4 == 0) && aligned(target_probs, 16) && (K == 0 || aligned(draft_probs, 16));
    const int occ = d.occ[vec ? 1 : 0];
    const uint64_t resident = (uint64_t)(occ > 0 ? occ : 1) * (uint64_t)d.cus;
    // batch tickets only when there are many per resident block: on small
    // launches a batch would serialise work that could run side by side
    a.batch = a.total >= 16u * resident ? kTicketBatch : (a.total >= 4u * resident ? 2u : 1u);
    const uint64_t blocks = (a.total + a.batch - 1) / a.batch;
    const unsigned grid = (unsigned)(resident < blocks ? resident : blocks);
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
